"""Writes prefill_asm.inc: the K loop of the prefill GEMM as gfx950 assembly.

The loop is emitted as the text of one inline-asm statement per workgroup
shape and scale mode (block scales, per-tensor scales).  gemm_kernels.hip prepares the operands
(tile origin, buffer descriptors, per-lane offsets) in C++ and hands them to
that statement; everything that touches the accumulators -- the copies into
LDS, the fragment reads, the MFMAs, the per-K-block scale fold and the bf16
stores -- is scheduled here instruction by instruction.

Why a generator: the instruction order is the performance.  The matrix unit
should never wait for the fragment reads or the copies, and the compiler's
scheduler, short of registers at 248 VGPRs, folds every partial product the
moment it is produced and waits on the matrix unit with s_nop.  Here each
K step is 4 fa MFMA slots (4 weight x fa activation fragments of the wave's
16 fa x 64 tile: 32 slots for 128 x 64, 16 for 64 x 64); memory operations
are spread over the slots, each partial is folded four MFMAs after it was
issued (the four folds go out ahead of the next MFMA's fragment wait), and
every LDS counter wait is computed from the issue order.

M0 is written by the copies (the LDS destination of buffer_load ... lds) and is
listed among the clobbers with the fixed registers, so the compiler keeps no
value of its own in it across the statement.  Labels end in %=, which the
compiler replaces by a number unique to each instance of the statement, so a
duplicated statement cannot redefine a label.

Run:  python gen_prefill_asm.py   (rewrites prefill_asm.inc next to it)
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "prefill_asm.inc")

# ---------------------------------------------------------------------------
# LDS layout (bytes from the kernel's LDS base), one per workgroup shape.
# gemm_kernels.hip takes its copy of these offsets from the #defines written
# below and static_asserts the ones it derives itself.
KB_GROUP = 4                      # K blocks per activation-scale copy
ROW_PAD = 16                      # bytes after every 8 operand rows
EP_PITCH = 144                    # bytes per staged output row (64 bf16 + 16 B pad)
EP_HALF = 64 * EP_PITCH           # one wave's staging area: 64 rows


class Layout:
    """One workgroup shape: nw waves on a tm x tn tile, wn = tn / 64 waves
    along N and wm = nw / wn along M, so a wave owns tm / wm rows (fa
    activation fragments) x 64 columns (4 weight fragments) and a K step is
    4 fa MFMA slots.

    LDS: operand stages (activation tm rows x 128 B, weight tn rows x 128 B,
    `stages` of each), then the two activation-scale group buffers (4 K
    blocks x tm rows each), then the weight-scale table [2][256].

    Operand rows are stored in units of 8 (1 KiB, what one copy instruction
    writes) followed by ROW_PAD bytes.  A fragment read takes one 16-byte
    chunk from each of 16 rows, and the LDS serves 16 lanes per cycle from
    64 four-byte banks (256 bytes).  Unpadded, rows r and r + 8 of a fragment
    start at the same bank, and the chunk swizzle (which keeps a lane's two
    chunks adjacent) cannot separate them, so every read took two cycles; the
    16-byte shift of the second unit puts them on different banks."""

    def __init__(self, nw, stages, tn=None, tm=256, pad=ROW_PAD, tag=""):
        self.nw, self.stages, self.tag = nw, stages, tag
        self.tm = tm                      # tile height (activation rows)
        self.tn = tn or 32 * nw           # tile width (weight rows)
        self.wn = self.tn // 64           # waves along N
        self.wm = nw // self.wn           # waves along M
        self.fa = tm // (16 * self.wm)    # activation fragments per wave
        self.q = 4 * self.fa              # MFMA slots per K step
        self.a_units, self.w_units = tm // 8, self.tn // 8
        self.sa_waves = tm // 64          # waves that copy the activation scales
        assert self.wm * self.wn == nw and self.fa in (4, 8) and nw % 2 == 0
        assert self.a_units % nw == 0 and self.w_units % nw == 0 and self.sa_waves <= nw
        self.unit = 1024 + pad            # 8 rows and the pad
        self.frag = 2 * self.unit         # 16 rows: one MFMA operand fragment
        a_bytes, w_bytes = self.a_units * self.unit, self.w_units * self.unit
        self.A = tuple(i * a_bytes for i in range(stages))
        w0 = stages * a_bytes
        self.W = tuple(w0 + i * w_bytes for i in range(stages))
        sa0 = w0 + stages * w_bytes
        self.SA = (sa0, sa0 + tm * KB_GROUP * 4)
        self.SW = self.SA[1] + tm * KB_GROUP * 4
        self.bytes = self.SW + 2 * 256 * 4
        assert self.bytes <= 160 * 1024
        assert nw * EP_HALF <= self.bytes     # the epilogue's staging areas


# ---------------------------------------------------------------------------
# Register map (fixed physical VGPRs; the operands handed in from C++ are
# allocated by the compiler above these).
ACC0 = 0                          # acc[i][j][r] = v[(i * 8 + j) * 4 + r], 128 VGPRs
FW0 = 128                         # weight fragments, two sets of 4 x 8 VGPRs
FA0 = 192                         # activation fragments, two buffers of 8 VGPRs
P0 = 208                          # six partial-product slots of 4 VGPRs
SC0 = 232                         # eight activation scales (times the weight scale)
SPREV = 240                       # scale of fragment 7 of the previous K step
SWN = 241                         # weight scale of the next K step
VCOPY = (242, 243)                # per-copy source offsets (alternating)
RDA_HI = 244                      # fragment-read base 64 KiB above rdA (a third stage)
# the same for rdW, in shapes with four activation fragments per wave (their
# accumulators leave acc(0, 4) .. unused)
RDW_HI = ACC0 + (0 * 8 + 4) * 4
NUM_FIXED_VGPR = 245
DS_OFFSET_MAX = 65535             # ds_read immediate offsets are 16-bit
# scalar scratch
S_KB, S_DK, S_DK4, S_T, S_R = "s84", "s85", "s86", "s87", "s88"
CLOBBER_SGPR = (84, 89)

# Workgroup shapes, by tag: (waves, LDS stages, tile width, tile height).
# Copy t of wave w carries tile rows 8 (w + nw t) .. + 7; the activation tile
# takes tm / (8 nw) copies per wave, the weight tile tn / (8 nw).
#   W8:  256 x 256, 8 waves of 128 x 64 (two per SIMD), two stages (the LDS
#        holds no third);
#   W8M: 128 x 256, 8 waves of 64 x 64 (two per SIMD), three stages, so the
#        copies run two K steps ahead; it alone carries the split-K hand-over.
SHAPES = {"W8": (8, 2, 256, 256), "W8M": (8, 3, 256, 128)}
SPLIT_SHAPE = "W8M"


def layout(tag):
    return Layout(*SHAPES[tag], tag=tag)


def copies(lay):
    """Order of one K block's copies: activation and weight interleaved."""
    na, nb = lay.a_units // lay.nw, lay.w_units // lay.nw
    a = [("A", t) for t in range(na)]
    w = [("W", t) for t in range(nb)]
    out = []
    for k in range(max(na, nb)):
        if k < na:
            out.append(a[k])
        if k < nb:
            out.append(w[k])
    return out

# partial-product slot of MFMA q (0..31) of a K step: every 5 consecutive
# MFMAs (cyclically, across K steps) use distinct slots, so a partial is
# folded 4 MFMAs after it was issued and its slot is free again by then.
SLOT_SEQS = {32: [0, 1, 2, 3, 4] * 5 + [0, 5, 1, 2, 3, 4, 5],
             16: [0, 1, 2, 3, 4] * 3 + [5]}
FOLD_LAG = 4
# A slot's four folds go out before its MFMA and ahead of the wait for its
# fragments, so the VALU works while the wave would otherwise wait on the
# LDS (timed against folds after the MFMA: 114.9 -> 108.6 us on the MLP-down
# shape, 61.7 -> 60.0 us at 4096^3, bit-identical output).
FOLDS_BEFORE = 4
# the step's copies start this many slots before its end.  With block
# scales right after its barrier (the barrier slot is Q - 6): timed against
# 4, 112.0 -> 110.8 us on the MLP-down shape and 1659 -> 1598 us on the
# large GEMM.  Scales constant along K keep 4 (95.2 against 98.8 us on the
# MLP-down shape).  Medians of interleaved runs.
COPY_LEAD = {True: 6, False: 4}   # by block scales or not
for _q, _seq in SLOT_SEQS.items():
    assert len(_seq) == _q
    _cyc = _seq + _seq[:FOLD_LAG]
    assert all(len(set(_cyc[q:q + FOLD_LAG + 1])) == FOLD_LAG + 1 for q in range(_q))

LGKM_MAX = 15                     # 4-bit counter on gfx9


def acc(i, j, r=0):
    return ACC0 + (i * 8 + j) * 4 + r


def vr(a, n):
    return f"v[{a}:{a + n - 1}]"


def fw(setn, i):
    return FW0 + 32 * setn + 8 * i


def fa(buf):
    return FA0 + 8 * buf


def pslot(q, nq=32):
    return P0 + 4 * SLOT_SEQS[nq][q % nq]


class Program:
    """Straight-line emitter with LDS-counter bookkeeping."""

    def __init__(self):
        self.lines = []
        self.issued = 0                 # LDS ops issued
        self.done_upto = 0              # LDS ops known complete (waited for)
        self.where = {}                 # key -> index (1-based) of its last LDS op
        self.max_out = 0
        self.vm_ops = []                # vector-memory ops issued: (key, every wave issues it)

    def emit(self, *ls):
        self.lines.extend(ls)

    def lds(self, key, *ls):
        self.emit(*ls)
        self.issued += len(ls)
        self.where[key] = self.issued
        self.max_out = max(self.max_out, self.issued - self.done_upto)
        assert self.issued - self.done_upto <= LGKM_MAX, ("too many LDS ops in flight", key)

    def need(self, *keys):
        idx = [self.where[k] for k in keys if k in self.where]
        if not idx:
            return
        last = max(idx)
        if last <= self.done_upto:
            return
        n = self.issued - last
        self.emit(f"s_waitcnt lgkmcnt({n})")
        self.done_upto = last

    def vm(self, key, *ls, every_wave=True):
        """A vector-memory op (a copy into LDS) tagged with key; every_wave
        False for ops some waves branch around."""
        self.emit(*ls)
        self.vm_ops.append((key, every_wave))

    def vm_wait_for(self, key):
        """Wait until the ops tagged key have completed.  Copies complete in
        issue order, so the ops every wave issued after key's last one may
        stay out (ops only some waves issue are not counted: a wave that
        issued them waits for more than it needs)."""
        last = max((i for i, (k, _) in enumerate(self.vm_ops) if k == key), default=None)
        n = 0 if last is None else sum(1 for _, e in self.vm_ops[last + 1:] if e)
        assert 0 <= n <= 63
        self.emit(f"s_waitcnt vmcnt({n})")

    def wait_all_lds(self):
        if self.done_upto < self.issued:
            self.emit("s_waitcnt lgkmcnt(0)")
            self.done_upto = self.issued


# ---------------------------------------------------------------------------
def frag_read(prog, key, dst, base, off):
    """The two 16-byte reads of a fragment at base operand + off; offsets
    past the 16-bit field go through RDA_HI / RDW_HI (64 KiB above the base)."""
    reg = f"%[{base}]"
    if off + 16 > DS_OFFSET_MAX:
        reg, off = f"v{RDA_HI if base == 'rdA' else RDW_HI}", off - 65536
    assert 0 <= off and off + 16 <= DS_OFFSET_MAX
    prog.lds(key, f"ds_read_b128 {vr(dst, 4)}, {reg} offset:{off}",
             f"ds_read_b128 {vr(dst + 4, 4)}, {reg} offset:{off + 16}")


def dma_copy(prog, lay, op, t, stage, k, blk):
    """Copy t (tile rows 8 (wave + nw t) .. + 7) of operand op, K block S_DK,
    into stage; the copy is tagged as part of K block blk.  The row offset
    t * nw * 8 * ld is added to the lane's offset in a VGPR (the descriptor's
    range check sees it: rows past M or N read zero); the K offset is the
    scalar offset."""
    base = (lay.A if op == "A" else lay.W)[stage] + t * lay.nw * lay.unit
    v = VCOPY[k % 2]
    if t == 0:
        prog.emit(f"v_mov_b32 v{v}, %[off{op}]")
    else:
        prog.emit(f"s_mul_i32 {S_R}, %[rs{op}], {t}",
                  f"v_add_u32 v{v}, {S_R}, %[off{op}]")
    prog.emit(f"s_add_u32 m0, %[wave1k], {base}", "s_nop 0")
    prog.vm(("blk", blk), f"buffer_load_dwordx4 v{v}, %[d{op}], {S_DK} offen lds")


_label = [0]


def dma_scale_group(prog, lay, buf, tag, first=None):
    """Waves 0 .. tm / 64 - 1: each lane copies the 16 bytes sa[row, g .. g + 3]
    of its row, g = min(first K block of the next group, KB - 4) (or `first`),
    into group buffer `buf`.  The other waves branch around."""
    _label[0] += 1
    skip = f"fp8pf_sa_{tag}_{_label[0]}_%="
    prog.emit("s_cmp_eq_u32 %[wsa], 0", f"s_cbranch_scc1 {skip}")
    if first is None:
        prog.emit(f"s_add_u32 {S_T}, {S_KB}, {KB_GROUP - 1}",
                  f"s_and_b32 {S_T}, {S_T}, {-KB_GROUP & 0xffffffff}",
                  f"s_min_u32 {S_T}, {S_T}, %[kbm4]",
                  f"s_lshl_b32 {S_T}, {S_T}, 2")
    else:
        prog.emit(f"s_mov_b32 {S_T}, {4 * first}")
    prog.emit(f"s_add_u32 m0, %[sam0], {lay.SA[buf] - lay.SA[0]}", "s_nop 0")
    prog.vm(("sa", buf), f"buffer_load_dwordx4 %[offSa], %[dSa], {S_T} offen lds",
            every_wave=lay.sa_waves == lay.nw)
    prog.emit(f"{skip}:")


def scale_reads(prog, key, kb_next, half):
    """ds_read2 of the lane's activation scales of K block kb_next: fragments
    4 half .. 4 half + 3 into SC0 + 4 half .. .  Entry (tile row r, block u)
    of a group buffer sits at 16 r + 4 u; the lane's rows are
    16 fa wm + 16 j + r16, so fragment j is 64 j + u dwords above the lane's
    base (one base per buffer and half: the read2 offsets are 8-bit), and the
    16 rows of a fragment fall on 16 distinct banks."""
    buf = (kb_next // KB_GROUP) % 2
    u = kb_next % KB_GROUP
    base = f"%[sc{'LH'[half]}{buf}]"
    ls = []
    for k in range(2):
        jj = 2 * k                       # fragment within the half
        ls.append(f"ds_read2_b32 {vr(SC0 + 4 * half + jj, 2)}, {base} "
                  f"offset0:{64 * jj + u} offset1:{64 * (jj + 1) + u}")
    prog.lds(key, *ls)


def set_dk(prog, ahead):
    """S_DK = 128 * min(kb + ahead, KB - 1), S_DK4 = 4 * the same block."""
    prog.emit(f"s_add_u32 {S_DK}, {S_KB}, {ahead}",
              f"s_min_u32 {S_DK}, {S_DK}, %[kbm1]",
              f"s_lshl_b32 {S_DK4}, {S_DK}, 2",
              f"s_lshl_b32 {S_DK}, {S_DK}, 7")


def loop_period(stages):
    """Steps after which the loop's code repeats: LDS stages cycle every
    `stages` steps, weight-fragment register sets every 2, activation-scale
    group buffers every 2 KB_GROUP."""
    from math import lcm
    return lcm(stages, 2, 2 * KB_GROUP)


def gen_loop(block, lay):
    """Steady-state K steps.  Returns the text of one period of consecutive
    steps (loop_period) as chunks of KB_GROUP steps, taken from the middle of
    a longer run so that the counter waits see the operations the previous
    steps left in flight."""
    nw, S, Q, FA = lay.nw, lay.stages, lay.q, lay.fa
    prog = Program()
    sched = {}

    def at(gslot, fn):
        sched.setdefault(gslot, []).append(fn)

    P = loop_period(S)
    nsteps = 3 * P
    # the barrier follows the last fragment read of the step's stage; the
    # next step's first reads follow it, five slots before their first use
    bar_slot = Q - 6
    lead = COPY_LEAD[block]
    assert Q - lead >= bar_slot          # a step's copies follow its barrier
    for st in range(nsteps):
        p = st % S                   # LDS stage of this step
        q = (st + 1) % S             # LDS stage of the next step
        rq = (st + 1) % 2            # weight-fragment register set of the next step
        base = Q * st
        # activation fragment j (1 .. FA - 1) of this step: after the last
        # MFMA of fragment j - 2 (same buffer), five slots before its first use
        for j in range(1, FA):
            at(base + 4 * j - 5, lambda st=st, j=j, p=p: frag_read(
                prog, ("fa", st, j), fa(j % 2), "rdA", lay.A[p] - lay.A[0] + j * lay.frag))

        def barrier(st=st):
            # this wave's reads of stage p are done and its copies of K block
            # st + 1 have landed; after the barrier every wave's have
            prog.wait_all_lds()
            prog.vm_wait_for(("blk", st + 1))
            prog.emit("s_barrier")
            set_dk(prog, S)
        at(base + bar_slot, barrier)
        at(base + Q - 5, lambda st=st, q=q, rq=rq: (
            frag_read(prog, ("fa", st + 1, 0), fa(0), "rdA", lay.A[q] - lay.A[0]),
            frag_read(prog, ("fw", st + 1, 0), fw(rq, 0), "rdW", lay.W[q] - lay.W[0])))
        for i in (1, 2, 3):
            at(base + Q - 5 + i, lambda st=st, q=q, rq=rq, i=i: frag_read(
                prog, ("fw", st + 1, i), fw(rq, i), "rdW", lay.W[q] - lay.W[0] + lay.frag * i))
        if block:
            # the next step's scales overwrite SC0 .. SC0 + 3.  With eight
            # fragments the folds still to come in this step read SC0 + 6, so
            # the reads go out at slot Q - 4; with four they read SC0 + 2
            # until slot Q - 1, so the reads wait for it (and the multiply
            # moves one slot later to give them the time).
            sc_slot, mul_slot = (Q - 4, 2) if FA == 8 else (Q - 1, 3)

            def scales_lo(st=st):
                prog.emit(f"v_mov_b32 v{SPREV}, v{SC0 + FA - 1}")
                scale_reads(prog, ("salo", st + 1), st + 1, 0)
                prog.emit("v_add_u32 %[swrd], 4, %[swrd]")
                prog.lds(("swn", st + 1), f"ds_read_b32 v{SWN}, %[swrd]")
            at(base + sc_slot, scales_lo)
            if FA == 8:
                # the second half at slot 4 of the next step (needed from slot 20)
                at(base + Q + 4, lambda st=st: scale_reads(prog, ("sahi", st + 1), st + 1, 1))

            def mul_lo(st=st):
                prog.need(("salo", st), ("swn", st))
                for r in range(4):
                    prog.emit(f"v_mul_f32_e32 v{SC0 + r}, v{SWN}, v{SC0 + r}")

            def mul_hi(st=st):
                prog.need(("sahi", st), ("swn", st))
                for r in range(4, 8):
                    prog.emit(f"v_mul_f32_e32 v{SC0 + r}, v{SWN}, v{SC0 + r}")
            at(base + mul_slot, mul_lo)
            if FA == 8:
                at(base + 12, mul_hi)
            if st % KB_GROUP == 1:
                nbuf = (st // KB_GROUP + 1) % 2
                at(base + Q - 2, lambda nbuf=nbuf: dma_scale_group(prog, lay, nbuf, f"blk{lay.tag}"))
        # copies of K block kb + S into this step's stage (released at the
        # barrier), one per slot from slot Q - lead on
        for k, (op, t) in enumerate(copies(lay)):
            at(base + Q - lead + k, lambda st=st, op=op, t=t, p=p, k=k: dma_copy(
                prog, lay, op, t, p, k, st + S))

    total = Q * nsteps
    marks = {}
    for gs in range(total):
        st, qq = divmod(gs, Q)
        if qq == 0:
            marks[st] = len(prog.lines)
        j, i = divmod(qq, 4)
        c = st % 2
        if block:
            pq = qq - FOLD_LAG
            jj, ii = divmod(pq % Q, 4)
            s = f"v{SC0 + jj}" if pq >= 0 else f"v{SPREV}"
            folds = [f"v_fmac_f32_e32 v{acc(ii, jj, r)}, {s}, v{pslot(pq, Q) + r}" for r in range(4)]
            nb = FOLDS_BEFORE
            # folds before the MFMA go out ahead of its fragment wait
            prog.emit(*folds[:nb])
            prog.need(("fa", st, j), ("fw", st, i))
            prog.emit(f"v_mfma_f32_16x16x128_f8f6f4 {vr(pslot(qq, Q), 4)}, {vr(fw(c, i), 8)}, "
                      f"{vr(fa(j % 2), 8)}, 0")
            prog.emit(*folds[nb:])
        else:
            prog.need(("fa", st, j), ("fw", st, i))
            prog.emit(f"v_mfma_f32_16x16x128_f8f6f4 {vr(acc(i, j), 4)}, {vr(fw(c, i), 8)}, "
                      f"{vr(fa(j % 2), 8)}, {vr(acc(i, j), 4)}")
        for fn in sched.get(gs, []):
            fn()
        if qq == Q - 1:
            prog.emit(f"s_add_u32 {S_KB}, {S_KB}, 1")
    marks[nsteps] = len(prog.lines)
    chunks = [prog.lines[marks[P + c]:marks[P + c + KB_GROUP]] for c in range(0, P, KB_GROUP)]
    return chunks, prog.max_out


def slot_words(lay):
    """s88 = byte offset of this wave's slot words: %[wsPart] is
    SPLIT_WORDS_BYTES + slot * split_part_bytes(lay), the words sit at
    16 slot."""
    shift = (split_part_bytes(lay) // 16).bit_length() - 1
    return [f"s_sub_u32 s88, %[wsPart], {SPLIT_WORDS_BYTES}", f"s_lshr_b32 s88, s88, {shift}"]


def split_quads(lay):
    """The wave's accumulator quads (4 VGPRs, acc(i, j)) in the order of its
    partial in the workspace: quad k of lane l at 1024 k + 16 l."""
    return [8 * i + j for i in range(4) for j in range(lay.fa)]


def split_part_bytes(lay):
    """One wave's fp32 partial: 16 fa x 64 accumulators."""
    return len(split_quads(lay)) * 1024


def gen_split_record(tag, lay):
    """Split-K launches: one lane records this half's XCD (+1) in the wave's
    workspace slot, word 2 + half, for the partner wave's hand-over."""
    skip = f"fp8pf_norec_{tag}_%="
    return ["s_cmp_eq_u32 %[xinfo], 0", f"s_cbranch_scc1 {skip}",
            "s_lshr_b32 s87, %[xinfo], 8",
            "s_lshl_b32 s87, s87, 2",
            "s_add_u32 s87, s87, 8",
            f"v_mov_b32 v{P0 + 1}, s87",
            XCC_READ,
            "s_add_u32 s86, s86, 1",
            f"v_mov_b32 v{P0}, s86",
            *slot_words(lay),
            "s_mov_b64 s[84:85], exec",
            "s_mov_b64 exec, 1",
            f"buffer_store_dword v{P0}, v{P0 + 1}, %[dWs], s88 offen sc0 sc1",
            "s_mov_b64 exec, s[84:85]",
            f"{skip}:"]


def gen_prologue(block, lay, tag="", split=False):
    nw, S = lay.nw, lay.stages
    # some scalar operands were just written by v_readfirstlane; VMEM reads of
    # an SGPR written by the VALU need wait states
    L = ["s_nop 7"]
    if split:
        L += gen_split_record(tag, lay)
    for i in range(4):
        for j in range(lay.fa):
            L += [f"v_mov_b32 v{acc(i, j, r)}, 0" for r in range(4)]
    if lay.A[-1] - lay.A[0] + lay.fa * lay.frag > DS_OFFSET_MAX:
        L.append(f"v_add_u32 v{RDA_HI}, 0x10000, %[rdA]")
    if lay.W[-1] - lay.W[0] + 4 * lay.frag > DS_OFFSET_MAX:
        assert lay.fa == 4
        L.append(f"v_add_u32 v{RDW_HI}, 0x10000, %[rdW]")
    if block:
        for k in range(24):
            L.append(f"v_mov_b32 v{P0 + k}, 0")
        L.append(f"v_mov_b32 v{SPREV}, 0")
        # weight-scale table: row b (this tile's weight blocks), blocks 64 (w % 4) + lane
        L += ["s_mov_b32 m0, %[swm0]", "s_nop 0", "buffer_load_dword %[offSw], %[dSw], 0 offen lds"]
    L.append(f"s_mov_b32 {S_KB}, 0")
    prog = Program()
    prog.emit(*L)
    if block:
        dma_scale_group(prog, lay, 0, f"pro{lay.tag}", first=0)
    # K blocks 0 .. S - 1 into stages 0 .. S - 1
    for stage in range(S):
        set_dk(prog, stage)
        for k, (op, t) in enumerate(copies(lay)):
            dma_copy(prog, lay, op, t, stage, k, stage)
    prog.vm_wait_for(("blk", 0))
    prog.emit("s_barrier")
    # leave S_DK on block S - 1: the first step re-issues the tail of that copy
    for i in range(4):
        frag_read(prog, None, fw(0, i), "rdW", i * lay.frag)
    frag_read(prog, None, fa(0), "rdA", 0)
    frag_read(prog, None, fa(1), "rdA", lay.frag)
    if block:
        prog.wait_all_lds()
        scale_reads(prog, None, 0, 0)
        if lay.fa == 8:
            scale_reads(prog, None, 0, 1)
        prog.emit(f"ds_read_b32 v{SWN}, %[swrd]")
    prog.emit("s_waitcnt lgkmcnt(0)")
    return prog.lines




SPLIT_WORDS_BYTES = 65536         # the slots' words come first: 16 bytes per slot
XCC_READ = "s_getreg_b32 s86, hwreg(HW_REG_XCC_ID, 0, 4)"   # this wave's XCD
SPIN_LIMIT = 1 << 22              # polls of the partner's flag (64-clock sleeps) before giving up


def gen_split_exchange(tag, lay):
    """Hand-over of a tile split in two along K (two workgroups, each half of
    the K blocks; a wave of one and the same wave of the other own the same
    (16 fa) x 64 outputs and share one workspace slot: four words -- arrival
    counter, flag, and the XCD records of the two halves -- and a fp32
    partial of 1 KiB per accumulator quad).  Each wave bumps the counter (one
    lane, an atomic add that returns the old count).  The first to arrive
    stores its accumulators (lane-major: quad k of lane l at 1024 k + 16 l,
    split_quads) and then writes the flag;
    the second polls the flag, adds the stored partial to its own and goes on
    to the bf16 stores.  fp32 addition commutes, so the sum does not depend
    on which of the two arrives first.

    Where the partial travels: every wave records its XCD (+1) when it
    starts (gen_split_record).  If the first finds its partner recorded on its own XCD, the two
    share an L2: the partial is stored plainly (the L1 writes through) and
    read back past the reader's L1 (sc0), flag 2.  Otherwise (partner on
    another XCD, or not started yet) it is written through and read past both
    L2s (sc0 sc1), flag 1.  The atomic, the records and the flag are
    system-coherent (sc0 sc1) and the partial's stores have completed
    (vmcnt 0) before the flag is written, so no cache is written back or
    invalidated as a whole.

    The first waits for nothing; the second waits only for a wave that has
    already finished its K loop, so the poll always ends (its limit only
    guards against words that were not cleared before the launch).
    %[xinfo] = 1 | (half << 8), or 0 when the launch does not split."""
    vt, vo, vl16 = P0, P0 + 1, P0 + 2
    tmp = FW0                          # 64 VGPRs: 16 quads of the partner's partial
    lab = {n: f"fp8pf_{n}_{tag}_%=" for n in
           ("done", "last", "spin", "ready", "nosplit", "fl2", "fflag", "l2h0", "l2h1", "addh0", "addh1")}
    words = slot_words(lay)
    quads = split_quads(lay)
    halves = [quads[h:h + 16] for h in range(0, len(quads), 16)]

    def one_lane(*ops):
        return ["s_mov_b64 exec, 1", *ops, "s_waitcnt vmcnt(0)", "s_mov_b64 exec, s[84:85]", "s_nop 1",
                f"v_readfirstlane_b32 s86, v{vt}", "s_nop 1"]

    def stores(bits):
        L = []
        for k, q in enumerate(quads):
            if k % 4 == 0:
                L.append(f"s_add_u32 s88, %[wsPart], {4096 * (k // 4)}")
            L.append(f"buffer_store_dwordx4 {vr(ACC0 + 4 * q, 4)}, v{vl16}, %[dWs], s88 offen "
                     f"offset:{1024 * (k % 4)}{bits}")
        return L

    def loads(h, bits):
        L = []
        for k in range(16 * h, 16 * h + len(halves[h])):
            if k % 4 == 0:
                L.append(f"s_add_u32 s88, %[wsPart], {4096 * (k // 4)}")
            L.append(f"buffer_load_dwordx4 {vr(tmp + 4 * (k % 16), 4)}, v{vl16}, %[dWs], s88 offen "
                     f"offset:{1024 * (k % 4)}{bits}")
        return L

    L = ["s_cmp_eq_u32 %[xinfo], 0", f"s_cbranch_scc1 {lab['nosplit']}",
         f"v_mbcnt_lo_u32_b32 v{vl16}, -1, 0",
         f"v_mbcnt_hi_u32_b32 v{vl16}, -1, v{vl16}",
         f"v_lshlrev_b32 v{vl16}, 4, v{vl16}",
         f"v_mov_b32 v{vo}, 0",
         "s_mov_b64 s[84:85], exec",
         *words]
    L += one_lane(f"v_mov_b32 v{vt}, 1",
                  f"buffer_atomic_add v{vt}, v{vo}, %[dWs], s88 offen sc0 sc1")
    L += ["s_cmp_eq_u32 s86, 0", f"s_cbranch_scc0 {lab['last']}"]
    # first to arrive: the partner's record sits at 12 - 4 half
    L += ["s_lshr_b32 s87, %[xinfo], 8",
          "s_lshl_b32 s87, s87, 2",
          "s_sub_u32 s87, 12, s87",
          f"v_mov_b32 v{vo}, s87"]
    L += one_lane(f"buffer_load_dword v{vt}, v{vo}, %[dWs], s88 offen sc0 sc1")
    L += [f"v_mov_b32 v{vo}, 0",
          XCC_READ.replace("s86", "s87"),
          "s_add_u32 s87, s87, 1",
          "s_cmp_eq_u32 s86, s87", f"s_cbranch_scc1 {lab['fl2']}"]
    L += stores(" sc0 sc1")
    L += ["s_mov_b32 s87, 1", f"s_branch {lab['fflag']}", f"{lab['fl2']}:"]
    L += stores("")
    L += ["s_mov_b32 s87, 2", f"{lab['fflag']}:",
          *words,
          "s_waitcnt vmcnt(0)",
          "s_mov_b64 exec, 1",
          f"v_mov_b32 v{vt}, s87",
          f"buffer_store_dword v{vt}, v{vo}, %[dWs], s88 offen offset:4 sc0 sc1",
          "s_waitcnt vmcnt(0)",
          "s_mov_b64 exec, s[84:85]",
          f"s_branch {lab['done']}"]
    # second to arrive: wait for the flag, then add the partial
    L += [f"{lab['last']}:", f"s_mov_b32 s87, {SPIN_LIMIT}", f"{lab['spin']}:"]
    L += one_lane(f"buffer_load_dword v{vt}, v{vo}, %[dWs], s88 offen offset:4 sc0 sc1")
    L += ["s_cmp_lg_u32 s86, 0", f"s_cbranch_scc1 {lab['ready']}",
          "s_sleep 1",
          "s_sub_u32 s87, s87, 1",
          "s_cmp_eq_u32 s87, 0",
          f"s_cbranch_scc0 {lab['spin']}",
          f"{lab['ready']}:"]
    for h in range(len(halves)):
        L += ["s_cmp_eq_u32 s86, 2", f"s_cbranch_scc1 {lab['l2h%d' % h]}"]
        L += loads(h, " sc0 sc1")
        L += [f"s_branch {lab['addh%d' % h]}", f"{lab['l2h%d' % h]}:"]
        L += loads(h, " sc0")
        L += [f"{lab['addh%d' % h]}:", "s_waitcnt vmcnt(0)"]
        for k, q in enumerate(halves[h]):
            for r in range(4):
                L.append(f"v_add_f32_e32 v{ACC0 + 4 * q + r}, v{ACC0 + 4 * q + r}, v{tmp + 4 * k + r}")
    L.append(f"{lab['nosplit']}:")
    return L


def gen_const_scales(lay):
    """Scales constant along K: out[m, n] = (sa[m] * sw[n]) * acc.  The
    lane's FA row scales (rows 16 FA wm + 16 j + r16) and 16 column scales
    (columns 64 wn + 16 i + 4 kg + r) come through range-checked descriptors
    (strides 0 give the per-tensor case)."""
    FA = lay.fa
    L = []
    sa_r, sw_r, vt = P0, P0 + 8, (SC0, SC0 + 1)
    n = 0
    for j in range(FA):
        t = vt[n % 2]
        n += 1
        if j == 0:
            L.append(f"v_mov_b32 v{t}, %[offSaR]")
        else:
            L += [f"s_mul_i32 {S_R}, %[sjA], {j}", f"v_add_u32 v{t}, {S_R}, %[offSaR]"]
        L.append(f"buffer_load_dword v{sa_r + j}, v{t}, %[dSaR], 0 offen")
    for i in range(4):
        for r in range(4):
            t = vt[n % 2]
            n += 1
            if i == 0 and r == 0:
                L.append(f"v_mov_b32 v{t}, %[offSwR]")
            else:
                L += [f"s_mul_i32 {S_R}, %[siW], {i}", f"s_mul_i32 {S_T}, %[srW], {r}",
                      f"s_add_u32 {S_R}, {S_R}, {S_T}", f"v_add_u32 v{t}, {S_R}, %[offSwR]"]
            L.append(f"buffer_load_dword v{sw_r + 4 * i + r}, v{t}, %[dSwR], 0 offen")
    L.append("s_waitcnt vmcnt(0)")
    for i in range(4):
        for j in range(FA):
            for r in range(4):
                L += [f"v_mul_f32_e32 v{vt[0]}, v{sa_r + j}, v{sw_r + 4 * i + r}",
                      f"v_mul_f32_e32 v{acc(i, j, r)}, v{vt[0]}, v{acc(i, j, r)}"]
    return L


def gen_epilogue(block, tag, lay, split=False):
    """Fold the last fragment (block scales), hand over a split tile's
    partial, apply scales constant along K, round to bf16 and store.  The wave's
    (16 fa) x 64 outputs go out in halves of 64 rows, each staged through LDS so that
    a lane stores 16 contiguous bytes and an instruction covers eight whole
    128-byte row segments (the MFMA layout gives a lane 4 adjacent values,
    i.e. 8-byte pieces of 16 rows).  The staged rows are 144 bytes apart:
    16 lanes writing 8 bytes each to 16 rows hit 16 distinct bank pairs."""
    # the last MFMAs' results are read by the VALU below: drain first
    nw, FA, Q = lay.nw, lay.fa, lay.q
    L = ["s_nop 7", "s_nop 7"]
    if block:
        # fold the last fragment of the last K step
        for q in range(Q - 4, Q):
            jj, ii = divmod(q, 4)
            for r in range(4):
                L.append(f"v_fmac_f32_e32 v{acc(ii, jj, r)}, v{SPREV}, v{pslot(q, Q) + r}")
    # every wave's copies and fragment reads are done: the stages are free
    L += ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier",
          "s_cmp_eq_u32 %[colok], 0", f"s_cbranch_scc1 fp8pf_done_{tag}_%="]
    if split:
        L += gen_split_exchange(tag, lay)
    if not block:
        # after the hand-over, so a split tile's two halves are scaled once
        # as their sum, like an unsplit tile's accumulator
        L += gen_const_scales(lay)
    vl, vt, vk, vw, vrd, vo = (FW0 + k for k in range(6))
    buf = FW0 + 8                      # 32 VGPRs of read-back data
    s_reg, s_ldo2, s_uni, s_step = S_KB, S_DK, S_DK4, S_T
    L += [f"v_mbcnt_lo_u32_b32 v{vl}, -1, 0",
          f"v_mbcnt_hi_u32_b32 v{vl}, -1, v{vl}",
          # staging area of this wave
          f"s_mul_i32 {s_reg}, %[wave], {EP_HALF}",
          f"s_add_u32 {s_reg}, {s_reg}, %[ldsb]",
          # write base: row r16, 8-byte piece kg
          f"v_and_b32 v{vt}, 15, v{vl}",
          f"v_mul_u32_u24 v{vt}, {EP_PITCH}, v{vt}",
          f"v_lshrrev_b32 v{vk}, 4, v{vl}",
          f"v_lshl_add_u32 v{vw}, v{vk}, 3, v{vt}",
          f"v_add_u32 v{vw}, {s_reg}, v{vw}",
          # read base: row lane / 8, 16-byte chunk lane % 8
          f"v_lshrrev_b32 v{vt}, 3, v{vl}",
          f"v_mul_u32_u24 v{vt}, {EP_PITCH}, v{vt}",
          f"v_and_b32 v{vk}, 7, v{vl}",
          f"v_lshl_add_u32 v{vrd}, v{vk}, 4, v{vt}",
          f"v_add_u32 v{vrd}, {s_reg}, v{vrd}",
          # store offset: row 16 FA wm + lane / 8, columns 64 wn + 8 (lane % 8)
          f"s_lshr_b32 {s_ldo2}, %[ldo16], 4",
          f"s_lshr_b32 {s_uni}, %[wave], {lay.wn.bit_length() - 1}",
          f"s_mul_i32 {s_uni}, {s_uni}, {16 * FA}",
          f"s_mul_i32 {s_uni}, {s_uni}, {s_ldo2}",
          f"s_and_b32 {s_step}, %[wave], {lay.wn - 1}",
          f"s_lshl_b32 {s_step}, {s_step}, 7",
          f"s_add_u32 {s_uni}, {s_uni}, {s_step}",
          f"v_lshrrev_b32 v{vt}, 3, v{vl}",
          f"v_mul_lo_u32 v{vt}, {s_ldo2}, v{vt}",
          f"v_lshl_add_u32 v{vo}, v{vk}, 4, v{vt}",
          f"v_add_u32 v{vo}, {s_uni}, v{vo}",
          f"s_lshr_b32 {s_step}, %[ldo16], 1"]          # 8 rows
    tmp = P0
    n = 0
    for h in range(FA // 4):
        for j in range(4 * h, 4 * h + 4):
            for i in range(4):
                t = tmp + 2 * (n % 12)
                off = (j - 4 * h) * 16 * EP_PITCH + i * 32
                L += [f"v_cvt_pk_bf16_f32 v{t}, v{acc(i, j, 0)}, v{acc(i, j, 1)}",
                      f"v_cvt_pk_bf16_f32 v{t + 1}, v{acc(i, j, 2)}, v{acc(i, j, 3)}",
                      f"ds_write_b64 v{vw}, {vr(t, 2)} offset:{off}"]
                n += 1
        for q in range(8):
            L.append(f"ds_read_b128 {vr(buf + 4 * q, 4)}, v{vrd} offset:{q * 8 * EP_PITCH}")
        L.append("s_waitcnt lgkmcnt(0)")
        for q in range(8):
            # a VALU write right after a 16-byte store of the registers it reads
            # needs a wait state
            L.append(f"buffer_store_dwordx4 {vr(buf + 4 * q, 4)}, v{vo}, %[dOut], 0 offen")
            L.append("s_nop 0")
            L.append(f"v_add_u32 v{vo}, {s_step}, v{vo}")
    L.append(f"fp8pf_done_{tag}_%=:")
    return L


def gen(block, shape="W8"):
    """KB must be a positive multiple of KB_GROUP (the caller checks).  Only
    SPLIT_SHAPE carries the split-K hand-over."""
    tag = ("blk" if block else "pt") + shape
    _label[0] = 0
    lay = layout(shape)
    split = shape == SPLIT_SHAPE
    chunks, max_out = gen_loop(block, lay)
    L = gen_prologue(block, lay, tag, split=split)
    L.append(f"fp8pf_loop_{tag}_%=:")
    for c, chunk in enumerate(chunks):
        L += chunk
        if c + 1 < len(chunks):              # K is any multiple of KB_GROUP blocks
            L += [f"s_cmp_eq_u32 {S_KB}, %[kb]", f"s_cbranch_scc1 fp8pf_tail_{tag}_%="]
    L += [f"s_cmp_lt_u32 {S_KB}, %[kb]", f"s_cbranch_scc1 fp8pf_loop_{tag}_%="]
    L.append(f"fp8pf_tail_{tag}_%=:")
    L += gen_epilogue(block, tag, lay, split=split)
    return L, max_out


def c_string(lines):
    return "\n".join(f'  "{l}\\n\\t"' for l in lines)


def main(path=OUT):
    out = ["// Generated by gen_prefill_asm.py; do not edit by hand.",
           "// K loop of gemm_prefill_kernel as gfx950 assembly (see that file).",
           "#pragma once", ""]
    for shape, block in [(t, b) for t in SHAPES for b in (True, False)]:
        lines, max_out = gen(block, shape)
        name = ("FP8_PREFILL_ASM_BLOCK" if block else "FP8_PREFILL_ASM_TENSOR") + f"_{shape}"
        out.append(f"// {len(lines)} lines; at most {max_out} LDS reads in flight")
        out.append(f"#define {name} \\")
        out.append(c_string(lines).replace("\n", " \\\n"))
        out.append("")
    vg = ", ".join(f'"v{k}"' for k in range(NUM_FIXED_VGPR))
    sg = ", ".join(f'"s{k}"' for k in range(*CLOBBER_SGPR))
    out.append(f'#define FP8_PREFILL_ASM_CLOBBERS {vg}, {sg}, "m0", "scc", "memory"')
    out.append(f"#define FP8_PREFILL_ASM_FIXED_VGPRS {NUM_FIXED_VGPR}")
    out.append(f"#define FP8_PREFILL_KB_GROUP {KB_GROUP}")
    out.append(f"#define FP8_PREFILL_SPLIT_WORDS_BYTES {SPLIT_WORDS_BYTES}")
    out.append(f"#define FP8_PREFILL_SPLIT_PART_BYTES {split_part_bytes(layout(SPLIT_SHAPE))}")
    for shape in SHAPES:
        lay = layout(shape)
        out.append(f"#define FP8_PREFILL_{shape}_WAVES {lay.nw}")
        out.append(f"#define FP8_PREFILL_{shape}_TM {lay.tm}")
        out.append(f"#define FP8_PREFILL_{shape}_TN {lay.tn}")
        out.append(f"#define FP8_PREFILL_{shape}_STAGES {lay.stages}")
        out.append(f"#define FP8_PREFILL_{shape}_LDS_UNIT {lay.unit}")
        out.append(f"#define FP8_PREFILL_{shape}_LDS_BYTES {lay.bytes}")
        out.append(f"#define FP8_PREFILL_{shape}_LDS_W {lay.W[0]}")
        out.append(f"#define FP8_PREFILL_{shape}_LDS_SA {lay.SA[0]}")
        out.append(f"#define FP8_PREFILL_{shape}_LDS_SA_GROUP_BYTES {lay.SA[1] - lay.SA[0]}")
        out.append(f"#define FP8_PREFILL_{shape}_LDS_SW {lay.SW}")
    text = "\n".join(out) + "\n"
    if path is None:
        return text
    with open(path, "w") as f:
        f.write(text)
    return text


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else OUT)
