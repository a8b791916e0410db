"""Writes prefill_asm.inc: the K loop of the prefill GEMM as gfx950 assembly.

The loop is emitted as the text of one inline-asm statement per scale mode
(block scales, per-tensor scales).  gemm_kernels.hip prepares the operands
(tile origin, buffer descriptors, per-lane offsets) in C++ and hands them to
that statement; everything that touches the accumulators -- the copies into
LDS, the fragment reads, the MFMAs, the per-K-block scale fold and the bf16
stores -- is scheduled here instruction by instruction.

Why a generator: the instruction order is the performance.  The matrix unit
should never wait for the fragment reads or the copies, and the compiler's
scheduler, short of registers at 248 VGPRs, folds every partial product the
moment it is produced and waits on the matrix unit with s_nop.  Here each
K step is 32 MFMA slots (4 weight x 8 activation fragments of the wave's
128 x 64 tile); memory operations are spread over the slots, each partial is
folded four MFMAs after it was issued, and every LDS counter wait is computed
from the issue order.

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
# LDS layout (bytes from the kernel's LDS base).  Kept in step with the
# constants in gemm_kernels.hip (kPfLds*), which static_asserts them.
A_STAGE = (0, 32768)              # 256 activation rows x 128 B per stage
W_STAGE = (65536, 98304)          # 256 weight rows x 128 B per stage
SA_GROUP = (131072, 135168)       # activation scales of 4 K blocks x 256 rows (permuted), x2
SW_TABLE = 139264                 # weight scales [2][256] of the tile's two weight blocks
LDS_BYTES = 141312
KB_GROUP = 4                      # K blocks per activation-scale copy

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
NUM_FIXED_VGPR = 244
# scalar scratch
S_KB, S_DK, S_DK4, S_T, S_R = "s84", "s85", "s86", "s87", "s88"
CLOBBER_SGPR = (84, 89)

# Workgroup shapes: NW waves in a 2 x (NW / 2) grid of 128 x 64 wave tiles,
# so the workgroup tile is 256 x (32 NW).  Copy t of wave w carries tile rows
# 8 (w + NW t) .. + 7; the activation tile takes 32 / NW copies per wave, the
# weight tile 4.
SHAPES = (8, 4)


def copies(nw):
    """Order of one K block's copies: activation and weight interleaved."""
    na = 32 // nw
    a = [("A", t) for t in range(na)]
    w = [("W", t) for t in range(4)]
    out = []
    for k in range(max(na, 4)):
        if k < na:
            out.append(a[k])
        if k < 4:
            out.append(w[k])
    return out

# partial-product slot of MFMA q (0..31) of a K step: every 5 consecutive
# MFMAs (cyclically, across K steps) use distinct slots, so a partial is
# folded 4 MFMAs after it was issued and its slot is free again by then.
SLOT_SEQ = [0, 1, 2, 3, 4] * 5 + [0, 5, 1, 2, 3, 4, 5]
FOLD_LAG = 4
assert len(SLOT_SEQ) == 32
_cyc = SLOT_SEQ + SLOT_SEQ[:FOLD_LAG]
assert all(len(set(_cyc[q:q + FOLD_LAG + 1])) == FOLD_LAG + 1 for q in range(32))

LGKM_MAX = 15                     # 4-bit counter on gfx9


def acc(i, j, r=0):
    return ACC0 + (i * 8 + j) * 4 + r


def vr(a, n):
    return f"v[{a}:{a + n - 1}]"


def fw(setn, i):
    return FW0 + 32 * setn + 8 * i


def fa(buf):
    return FA0 + 8 * buf


def pslot(q):
    return P0 + 4 * SLOT_SEQ[q % 32]


class Program:
    """Straight-line emitter with LDS-counter bookkeeping."""

    def __init__(self):
        self.lines = []
        self.issued = 0                 # LDS ops issued
        self.done_upto = 0              # LDS ops known complete (waited for)
        self.where = {}                 # key -> index (1-based) of its last LDS op
        self.max_out = 0

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

    def wait_all_lds(self):
        if self.done_upto < self.issued:
            self.emit("s_waitcnt lgkmcnt(0)")
            self.done_upto = self.issued


# ---------------------------------------------------------------------------
def frag_read(prog, key, dst, base, off):
    prog.lds(key, f"ds_read_b128 {vr(dst, 4)}, %[{base}] offset:{off}",
             f"ds_read_b128 {vr(dst + 4, 4)}, %[{base}] offset:{off + 16}")


def dma_copy(prog, op, t, stage, nw, k):
    """Copy t (tile rows 8 (wave + nw t) .. + 7) of operand op, K block S_DK,
    into stage.  The row offset t * nw * 8 * ld is added to the lane's offset
    in a VGPR (the descriptor's range check sees it: rows past M or N read
    zero); the K offset is the scalar offset."""
    base = (A_STAGE if op == "A" else W_STAGE)[stage] + t * nw * 1024
    v = VCOPY[k % 2]
    if t == 0:
        prog.emit(f"v_mov_b32 v{v}, %[off{op}]")
    else:
        prog.emit(f"s_mul_i32 {S_R}, %[rs{op}], {t}",
                  f"v_add_u32 v{v}, {S_R}, %[off{op}]")
    prog.emit(f"s_add_u32 m0, %[wave1k], {base}",
              "s_nop 0",
              f"buffer_load_dwordx4 v{v}, %[d{op}], {S_DK} offen lds")


_label = [0]


def dma_scale_group(prog, buf, tag, first=None):
    """Waves 0-3: each lane copies the 16 bytes sa[row, g .. g + 3] of its row,
    g = min(first K block of the next group, KB - 4) (or `first`), into group
    buffer `buf`.  Waves 4-7 branch around."""
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
    prog.emit(f"s_add_u32 m0, %[sam0], {SA_GROUP[buf] - SA_GROUP[0]}",
              "s_nop 0",
              f"buffer_load_dwordx4 %[offSa], %[dSa], {S_T} offen lds",
              f"{skip}:")


def scale_reads(prog, key, kb_next, half):
    """ds_read2 of the lane's activation scales of K block kb_next: fragments
    4 half .. 4 half + 3 into SC0 + 4 half .. .  Entry (tile row r, block u)
    of a group buffer sits at 16 r + 4 u; the lane's rows are
    128 wm + 16 j + r16, so fragment j is 64 j + u dwords above the lane's
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


def gen_loop(block, nw):
    """Steady-state K steps.  Returns the text of 2 x KB_GROUP consecutive
    steps as two halves (K blocks 0 .. 7 mod 8: LDS stages alternate every
    step, activation-scale group buffers every four), taken from the middle
    of a longer run so that the counter waits see the operations the
    previous steps left in flight."""
    prog = Program()
    sched = {}

    def at(gslot, fn):
        sched.setdefault(gslot, []).append(fn)

    nsteps = 6 * KB_GROUP
    bar_slot = 26
    for st in range(nsteps):
        p = st % 2                   # LDS stage of this step = weight-fragment set
        base = 32 * st
        # activation fragment j (1..7) of this step: after the last MFMA of
        # fragment j - 2 (same buffer), five slots before its first use
        for j in range(1, 8):
            at(base + 4 * j - 5, lambda st=st, j=j, p=p: frag_read(
                prog, ("fa", st, j), fa(j % 2), "rdA", A_STAGE[p] - A_STAGE[0] + j * 2048))

        def barrier(st=st):
            prog.wait_all_lds()
            prog.emit("s_waitcnt vmcnt(0)", "s_barrier")
            set_dk(prog, 2)
        at(base + bar_slot, barrier)
        q = 1 - p
        at(base + 27, lambda st=st, q=q: (
            frag_read(prog, ("fa", st + 1, 0), fa(0), "rdA", A_STAGE[q] - A_STAGE[0]),
            frag_read(prog, ("fw", st + 1, 0), fw(q, 0), "rdW", W_STAGE[q] - W_STAGE[0])))
        at(base + 28, lambda st=st, q=q: frag_read(
            prog, ("fw", st + 1, 1), fw(q, 1), "rdW", W_STAGE[q] - W_STAGE[0] + 2048))
        at(base + 29, lambda st=st, q=q: frag_read(
            prog, ("fw", st + 1, 2), fw(q, 2), "rdW", W_STAGE[q] - W_STAGE[0] + 4096))
        at(base + 30, lambda st=st, q=q: frag_read(
            prog, ("fw", st + 1, 3), fw(q, 3), "rdW", W_STAGE[q] - W_STAGE[0] + 6144))
        if block:
            def scales_lo(st=st):
                prog.emit(f"v_mov_b32 v{SPREV}, v{SC0 + 7}")
                scale_reads(prog, ("salo", st + 1), st + 1, 0)
                prog.emit("v_add_u32 %[swrd], 4, %[swrd]")
                prog.lds(("swn", st + 1), f"ds_read_b32 v{SWN}, %[swrd]")
            at(base + 28, scales_lo)
            # the second half at slot 4 of the next step (needed from slot 20)
            at(base + 32 + 4, lambda st=st: scale_reads(prog, ("sahi", st + 1), st + 1, 1))

            def mul_lo(st=st):
                prog.need(("salo", st), ("swn", st))
                for r in range(4):
                    prog.emit(f"v_mul_f32_e32 v{SC0 + r}, v{SWN}, v{SC0 + r}")

            def mul_hi(st=st):
                prog.need(("sahi", st), ("swn", st))
                for r in range(4, 8):
                    prog.emit(f"v_mul_f32_e32 v{SC0 + r}, v{SWN}, v{SC0 + r}")
            at(base + 2, mul_lo)
            at(base + 12, mul_hi)
            if st % KB_GROUP == 1:
                nbuf = (st // KB_GROUP + 1) % 2
                at(base + 30, lambda nbuf=nbuf: dma_scale_group(prog, nbuf, f"blk{nw}"))
        # copies of K block kb + 2 into this step's stage (released at the
        # barrier), one per slot from slot 28 on
        for k, (op, t) in enumerate(copies(nw)):
            at(base + 28 + k, lambda op=op, t=t, p=p, k=k: dma_copy(prog, op, t, p, nw, k))

    total = 32 * nsteps
    marks = {}
    for gs in range(total):
        st, qq = divmod(gs, 32)
        if qq == 0:
            marks[st] = len(prog.lines)
        j, i = divmod(qq, 4)
        c = st % 2
        prog.need(("fa", st, j), ("fw", st, i))
        if block:
            prog.emit(f"v_mfma_f32_16x16x128_f8f6f4 {vr(pslot(qq), 4)}, {vr(fw(c, i), 8)}, "
                      f"{vr(fa(j % 2), 8)}, 0")
            pq = qq - FOLD_LAG
            jj, ii = divmod(pq % 32, 4)
            s = f"v{SC0 + jj}" if pq >= 0 else f"v{SPREV}"
            for r in range(4):
                prog.emit(f"v_fmac_f32_e32 v{acc(ii, jj, r)}, {s}, v{pslot(pq) + r}")
        else:
            prog.emit(f"v_mfma_f32_16x16x128_f8f6f4 {vr(acc(i, j), 4)}, {vr(fw(c, i), 8)}, "
                      f"{vr(fa(j % 2), 8)}, {vr(acc(i, j), 4)}")
        for fn in sched.get(gs, []):
            fn()
        if qq == 31:
            prog.emit(f"s_add_u32 {S_KB}, {S_KB}, 1")
    marks[nsteps] = len(prog.lines)
    first = prog.lines[marks[2 * KB_GROUP]:marks[3 * KB_GROUP]]
    second = prog.lines[marks[3 * KB_GROUP]:marks[4 * KB_GROUP]]
    return first, second, prog.max_out


def gen_prologue(block, nw):
    # some scalar operands were just written by v_readfirstlane; VMEM reads of
    # an SGPR written by the VALU need wait states
    L = ["s_nop 7"]
    for k in range(128):
        L.append(f"v_mov_b32 v{ACC0 + k}, 0")
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
        dma_scale_group(prog, 0, f"pro{nw}", first=0)
    # K blocks 0 and 1 into stages 0 and 1
    for stage, ahead in ((0, 0), (1, 1)):
        set_dk(prog, ahead)
        for k, (op, t) in enumerate(copies(nw)):
            dma_copy(prog, op, t, stage, nw, k)
    prog.emit(f"s_waitcnt vmcnt({len(copies(nw))})", "s_barrier")
    # leave S_DK on block 1: the first step re-issues the tail of that copy
    for i in range(4):
        frag_read(prog, None, fw(0, i), "rdW", i * 2048)
    frag_read(prog, None, fa(0), "rdA", 0)
    frag_read(prog, None, fa(1), "rdA", 2048)
    if block:
        prog.wait_all_lds()
        scale_reads(prog, None, 0, 0)
        scale_reads(prog, None, 0, 1)
        prog.emit(f"ds_read_b32 v{SWN}, %[swrd]")
    prog.emit("s_waitcnt lgkmcnt(0)")
    return prog.lines


EP_PITCH = 144                    # bytes per staged output row (64 bf16 + 16 B pad)
EP_HALF = 64 * EP_PITCH           # one wave's staging area: 64 rows


def gen_epilogue(block, tag, nw):
    """Fold the last fragment, round to bf16 and store.  The wave's 128 x 64
    outputs go out in two halves of 64 rows, each staged through LDS so that
    a lane stores 16 contiguous bytes and an instruction covers eight whole
    128-byte row segments (the MFMA layout gives a lane 4 adjacent values,
    i.e. 8-byte pieces of 16 rows).  The staged rows are 144 bytes apart:
    16 lanes writing 8 bytes each to 16 rows hit 16 distinct bank pairs."""
    # the last MFMAs' results are read by the VALU below: drain first
    L = ["s_nop 7", "s_nop 7"]
    if block:
        # fold fragment 7 of the last K step
        for q in range(28, 32):
            jj, ii = divmod(q, 4)
            for r in range(4):
                L.append(f"v_fmac_f32_e32 v{acc(ii, jj, r)}, v{SPREV}, v{pslot(q) + r}")
    else:
        # scales constant along K: out[m, n] = (sa[m] * sw[n]) * acc.  The
        # lane's 8 row scales (rows 128 wm + 16 j + r16) and 16 column scales
        # (columns 64 wn + 16 i + 4 kg + r) come through range-checked
        # descriptors (strides 0 give the per-tensor case).
        sa_r, sw_r, vt = P0, P0 + 8, (SC0, SC0 + 1)
        n = 0
        for j in range(8):
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
            for j in range(8):
                for r in range(4):
                    L += [f"v_mul_f32_e32 v{vt[0]}, v{sa_r + j}, v{sw_r + 4 * i + r}",
                          f"v_mul_f32_e32 v{acc(i, j, r)}, v{vt[0]}, v{acc(i, j, r)}"]
    # every wave's copies and fragment reads are done: the stages are free
    L += ["s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier",
          "s_cmp_eq_u32 %[colok], 0", f"s_cbranch_scc1 fp8pf_done_{tag}_%="]
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
          # store offset: row 128 wm + lane / 8, columns 64 wn + 8 (lane % 8)
          f"s_lshr_b32 {s_ldo2}, %[ldo16], 4",
          f"s_lshr_b32 {s_uni}, %[wave], {(nw // 2).bit_length() - 1}",
          f"s_mul_i32 {s_uni}, {s_uni}, 128",
          f"s_mul_i32 {s_uni}, {s_uni}, {s_ldo2}",
          f"s_and_b32 {s_step}, %[wave], {nw // 2 - 1}",
          f"s_lshl_b32 {s_step}, {s_step}, 7",
          f"s_add_u32 {s_uni}, {s_uni}, {s_step}",
          f"v_lshrrev_b32 v{vt}, 3, v{vl}",
          f"v_mul_lo_u32 v{vt}, {s_ldo2}, v{vt}",
          f"v_lshl_add_u32 v{vo}, v{vk}, 4, v{vt}",
          f"v_add_u32 v{vo}, {s_uni}, v{vo}",
          f"s_lshr_b32 {s_step}, %[ldo16], 1"]          # 8 rows
    tmp = P0
    n = 0
    for h in range(2):
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


def gen(block, nw=8):
    """KB must be a positive multiple of KB_GROUP (the caller checks)."""
    tag = ("blk" if block else "pt") + str(nw)
    _label[0] = 0
    first, second, max_out = gen_loop(block, nw)
    L = gen_prologue(block, nw)
    L.append(f"fp8pf_loop_{tag}_%=:")
    L += first
    L += [f"s_cmp_eq_u32 {S_KB}, %[kb]", f"s_cbranch_scc1 fp8pf_tail_{tag}_%="]
    L += second
    L += [f"s_cmp_lt_u32 {S_KB}, %[kb]", f"s_cbranch_scc1 fp8pf_loop_{tag}_%="]
    L.append(f"fp8pf_tail_{tag}_%=:")
    L += gen_epilogue(block, tag, nw)
    return L, max_out


def c_string(lines):
    return "\n".join(f'  "{l}\\n\\t"' for l in lines)


def main(path=OUT):
    out = ["// Generated by gen_prefill_asm.py; do not edit by hand.",
           "// K loop of gemm_prefill_kernel as gfx950 assembly (see that file).",
           "#pragma once", ""]
    for nw, block in [(nw, b) for nw in SHAPES for b in (True, False)]:
        lines, max_out = gen(block, nw)
        name = ("FP8_PREFILL_ASM_BLOCK" if block else "FP8_PREFILL_ASM_TENSOR") + f"_W{nw}"
        out.append(f"// {len(lines)} lines; at most {max_out} LDS reads in flight")
        out.append(f"#define {name} \\")
        out.append(c_string(lines).replace("\n", " \\\n"))
        out.append("")
    vg = ", ".join(f'"v{k}"' for k in range(NUM_FIXED_VGPR))
    sg = ", ".join(f'"s{k}"' for k in range(*CLOBBER_SGPR))
    out.append(f'#define FP8_PREFILL_ASM_CLOBBERS {vg}, {sg}, "m0", "scc", "memory"')
    out.append(f"#define FP8_PREFILL_ASM_FIXED_VGPRS {NUM_FIXED_VGPR}")
    out.append(f"#define FP8_PREFILL_LDS_BYTES {LDS_BYTES}")
    out.append(f"#define FP8_PREFILL_LDS_SA {SA_GROUP[0]}")
    out.append(f"#define FP8_PREFILL_LDS_SA_GROUP_BYTES {SA_GROUP[1] - SA_GROUP[0]}")
    out.append(f"#define FP8_PREFILL_LDS_SW {SW_TABLE}")
    out.append(f"#define FP8_PREFILL_KB_GROUP {KB_GROUP}")
    out.append(f"#define FP8_PREFILL_LDS_W {W_STAGE[0]}")
    text = "\n".join(out) + "\n"
    if path is None:
        return text
    with open(path, "w") as f:
        f.write(text)
    return text


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else OUT)
