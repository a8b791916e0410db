"""The committed K-loop assembly (prefill_asm.inc) is what its generator writes.

gen_prefill_asm.py asserts its own scheduling invariants while it runs
(partial-product slots never reused before they are folded, never more than
15 LDS reads in flight for the 4-bit counter, fragment offsets inside the
16-bit field); this test runs it and checks that the include file the
library is built from is its current output, that each shape's LDS layout
fits, and that every copy a barrier waits for is counted."""
import importlib.util
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "fp8_w8a8_block_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_prefill_asm",
                                                  os.path.join(CSRC, "gen_prefill_asm.py"))
    g = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(g)
    return g


def test_include_is_generator_output():
    g = _gen()
    text = g.main(None)
    with open(os.path.join(CSRC, "prefill_asm.inc")) as f:
        assert f.read() == text, "prefill_asm.inc is stale: run gen_prefill_asm.py"


def _all(g):
    return [(tag, b) for tag in g.SHAPES for b in (True, False)]


def test_fixed_registers_and_lds_fit():
    g = _gen()
    assert g.NUM_FIXED_VGPR + 11 <= 256          # fixed map plus the C++ operands
    for tag in g.SHAPES:
        lay = g.layout(tag)
        assert lay.bytes <= 160 * 1024
        # stages, then the scale groups and the table, none overlapping
        assert lay.A[-1] + lay.a_units * lay.unit <= lay.W[0]
        assert lay.W[-1] + lay.w_units * lay.unit <= lay.SA[0]
        assert lay.SA[1] + lay.tm * g.KB_GROUP * 4 <= lay.SW and lay.SW + 2048 == lay.bytes
    for tag, block in _all(g):
        lay = g.layout(tag)
        lines, max_out = g.gen(block, tag)
        assert max_out <= 15
        regs = [int(m) for l in lines for m in re.findall(r"\bv(\d+)\b", l)]
        regs += [int(b) for l in lines for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", l)]
        assert max(regs) < g.NUM_FIXED_VGPR
        if lay.fa == 4:
            # accumulators of fragments 4-7 are free: the high weight base
            # lives there and nothing else writes it
            used = {g.acc(i, j, r) for i in range(4) for j in range(4) for r in range(4)}
            assert g.RDW_HI not in used
            writes = [l for l in lines if re.match(rf"\S+ v{g.RDW_HI}\b", l)
                      or re.search(rf"v\[(\d+):(\d+)\]", l.split(",")[0]) and
                      any(int(a) <= g.RDW_HI <= int(b)
                          for a, b in re.findall(r"v\[(\d+):(\d+)\]", l.split(",")[0]))]
            assert all(l.startswith("v_add_u32") for l in writes), writes


def test_every_lds_wait_names_a_smaller_count():
    # counts in s_waitcnt lgkmcnt(n) stay encodable (4 bits)
    g = _gen()
    for tag, block in _all(g):
        lines, _ = g.gen(block, tag)
        for l in lines:
            m = re.match(r"s_waitcnt lgkmcnt\((\d+)\)", l)
            if m:
                assert int(m.group(1)) <= 15


def test_barriers_wait_for_the_next_block():
    # with S stages, the copies a step issues are for block kb + S and its
    # barrier must leave at most the copies issued after block kb + 1 in
    # flight: none with two stages, one step's copies (plus at most one
    # scale copy) with three
    g = _gen()
    for tag, block in _all(g):
        lay = g.layout(tag)
        lines, _ = g.gen(block, tag)
        # the waits right before a barrier: the prologue's, then one per step
        waits = [int(m.group(1)) for l, nxt in zip(lines, lines[1:]) if nxt == "s_barrier"
                 for m in [re.fullmatch(r"s_waitcnt vmcnt\((\d+)\)", l)] if m]
        n = len(g.copies(lay))
        loop = waits[1:]
        assert len(loop) == g.loop_period(lay.stages)
        if lay.stages == 2:
            assert set(loop) == {0}
        else:
            assert set(loop) <= {n, n + 1} and waits[0] == (lay.stages - 1) * n


def _bank_groups(addrs):
    """16-byte bank groups (of the 16 in 64 four-byte banks) of 16 lanes'
    16-byte accesses."""
    return [(a // 16) % 16 for a in addrs]


def test_fragment_reads_are_conflict_free():
    # the LDS serves a ds_read_b128 16 lanes at a time from 64 four-byte
    # banks; each lane of a 16-lane group reads one 16-byte chunk of its own
    # row, and the 16 chunks must fall on 16 distinct bank groups.  Lane
    # (r16, kg) of a wave reads row 16 j + r16 of its rows, chunks 2 kg and
    # 2 kg + 1, stored at positions XOR-swizzled by 2 ((row >> 1) & 3).
    g = _gen()

    def swz_pair(r):
        return 2 * ((r >> 1) & 3)

    for tag in g.SHAPES:
        lay = g.layout(tag)
        for j in range(lay.fa):                              # fragment of the wave
            for half in range(2):                            # first or second ds_read_b128
                for kg in range(4):                          # 16-lane group
                    addrs = []
                    for r16 in range(16):
                        row = 16 * j + r16
                        pos = (2 * kg) ^ swz_pair(r16)
                        addrs.append((row // 8) * lay.unit + (row % 8) * 128 + pos * 16 + 16 * half)
                    assert len(set(_bank_groups(addrs))) == 16, (tag, j, half, kg)
        # the unpadded layout meets every bank twice
        flat = g.Layout(*g.SHAPES[tag], pad=0)
        addrs = [(r // 8) * flat.unit + (r % 8) * 128 + swz_pair(r) * 16 for r in range(16)]
        assert len(set(_bank_groups(addrs))) == 8


def test_copies_land_where_fragments_are_read():
    # copy t of wave w writes tile rows 8 (w + NW t) .. + 7 as one 1 KiB unit
    # at stage + (w + NW t) * unit; fragment j of wave row wm (wave column
    # wn) starts at unit 2 fa wm + 2 j (8 wn + 2 j): the two addressings
    # agree for every activation (weight) row
    g = _gen()
    for tag in g.SHAPES:
        lay = g.layout(tag)
        for units, rows_per_wave in ((lay.a_units, 16 * lay.fa), (lay.w_units, 64)):
            seen = set()
            for w in range(lay.nw):
                for t in range(units // lay.nw):
                    u = w + lay.nw * t
                    for r in range(8):
                        row = 8 * u + r
                        wr, j, r16 = row // rows_per_wave, (row % rows_per_wave) // 16, row % 16
                        by_read = (wr * (rows_per_wave // 8) * lay.unit + j * lay.frag +
                                   (r16 // 8) * lay.unit + (r16 % 8) * 128)
                        by_copy = u * lay.unit + r * 128
                        assert by_read == by_copy
                        seen.add(row)
            assert seen == set(range(8 * units))
        assert lay.A[1] - lay.A[0] == lay.a_units * lay.unit
        assert lay.W[0] == lay.stages * lay.a_units * lay.unit
        assert 8 * lay.a_units == lay.tm and 8 * lay.w_units == lay.tn


def test_fragment_reads_stay_in_their_stage():
    # every ds_read_b128 of an operand fragment, for every wave and lane,
    # lies inside one stage of that operand: rdA / rdW are the lane's bases
    # (wave row / column offset plus the in-fragment row and chunk), the high
    # bases 64 KiB above them
    g = _gen()
    for tag, block in _all(g):
        lay = g.layout(tag)
        lines, _ = g.gen(block, tag)
        rd_rows = [(r16 >> 3) * lay.unit + (r16 & 7) * 128 + 16 * (((2 * kg) ^ (2 * ((r16 >> 1) & 3))))
                   for r16 in range(16) for kg in range(4)]
        bases = {"rdA": [wm * 2 * lay.fa * lay.unit for wm in range(lay.wm)],
                 "rdW": [lay.W[0] + wn * 8 * lay.unit for wn in range(lay.wn)]}
        regions = {"rdA": [(a, a + lay.a_units * lay.unit) for a in lay.A],
                   "rdW": [(w, w + lay.w_units * lay.unit) for w in lay.W]}
        n = 0
        for l in lines:
            m = re.fullmatch(r"ds_read_b128 v\[\d+:\d+\], (%\[rd[AW]\]|v\d+) offset:(\d+)", l)
            if not m:
                continue
            reg, off = m.group(1), int(m.group(2))
            if reg.startswith("%"):
                op, hi = reg[2:5], 0
            elif int(reg[1:]) in (g.RDA_HI, g.RDW_HI):
                op, hi = ("rdA" if int(reg[1:]) == g.RDA_HI else "rdW"), 65536
            else:
                continue                # the epilogue's read-back of staged outputs
            for b in bases[op]:
                for rr in rd_rows:
                    addr = b + rr + hi + off
                    assert any(lo <= addr and addr + 16 <= up for lo, up in regions[op]), (tag, l)
            n += 1
        assert n > 0


def test_split_handover_stays_in_its_slot():
    # every workspace access of the split-K hand-over lies inside the wave's
    # slot: its four words (16 bytes at 16 slot) and its partial (quad k of
    # lane l at 1024 k + 16 l, one quad per accumulator quad); only the split
    # shape hands over, and every accumulator it holds travels
    g = _gen()
    lay = g.layout(g.SPLIT_SHAPE)
    part = g.split_part_bytes(lay)
    quads = g.split_quads(lay)
    assert part == 16 * lay.fa * 64 * 4 and len(set(quads)) == 4 * lay.fa
    assert {g.acc(i, j) for i in range(4) for j in range(lay.fa)} == {g.ACC0 + 4 * q for q in quads}
    for block in (True, False):
        lines, _ = g.gen(block, g.SPLIT_SHAPE)
        base = None
        seen = 0
        for l, nxt in zip(lines, lines[1:] + [""]):
            m = re.fullmatch(r"s_add_u32 s88, %\[wsPart\], (\d+)", l)
            if m:
                base = int(m.group(1))
                assert base % 4096 == 0 and base < part
            if l == f"s_sub_u32 s88, %[wsPart], {g.SPLIT_WORDS_BYTES}":
                # 16 bytes of words per slot of `part` bytes
                assert nxt == f"s_lshr_b32 s88, s88, {(part // 16).bit_length() - 1}"
                assert 1 << ((part // 16).bit_length() - 1) == part // 16
                base = "words"
            if "%[dWs]" in l:
                seen += 1
                off = int(re.search(r"offset:(\d+)", l).group(1)) if "offset:" in l else 0
                assert "s88" in l and base is not None
                if base == "words":                          # the words (voffset 0 or 8 / 12)
                    assert off in (0, 4)
                else:                                        # a 16-byte quad, lane offset <= 1008
                    assert l.startswith(("buffer_load_dwordx4", "buffer_store_dwordx4"))
                    assert base + off + 1008 + 16 <= part
        n = len(quads)
        assert seen == 1 + 1 + 1 + 2 * n + 1 + 1 + 2 * n      # record, atomic, partner, stores, flag, poll, loads
        for tag in g.SHAPES:
            if tag != g.SPLIT_SHAPE:
                assert not any("%[dWs]" in l or "%[xinfo]" in l for l in g.gen(block, tag)[0])


def test_scales_are_not_overwritten_before_their_last_fold():
    # block scales: the reads of the next step's activation scales (ds_read2
    # into SC0 + k) must come after the last fold of this step that reads
    # SC0 + k, and the fold must not read SC0 + k again before the new value
    # has been multiplied by the weight scale (v_mul_f32 SC0 + k, SWN, ...)
    g = _gen()
    for tag in g.SHAPES:
        lines, _ = g.gen(True, tag)
        pending = set()                 # SC registers loaded but not yet scaled
        for l in lines:
            m = re.match(r"ds_read2_b32 v\[(\d+):(\d+)\]", l)
            if m:
                pending |= set(range(int(m.group(1)), int(m.group(2)) + 1))
                continue
            m = re.match(rf"v_mul_f32_e32 v(\d+), v{g.SWN}, v(\d+)", l)
            if m and m.group(1) == m.group(2):
                pending.discard(int(m.group(1)))
                continue
            m = re.match(r"v_fmac_f32_e32 v\d+, v(\d+), ", l)
            if m:
                assert int(m.group(1)) not in pending, (tag, l)


def test_no_copy_overwrites_a_stage_before_every_wave_has_read_it():
    # LDS write-after-read across waves: a copy into stage p (its m0 base
    # names the stage) must come after a barrier that follows this wave's
    # last fragment read of stage p (the read's offset names the stage)
    g = _gen()
    for tag, block in _all(g):
        lay = g.layout(tag)
        a_bytes, w_bytes = lay.a_units * lay.unit, lay.w_units * lay.unit
        lines = [l for c in g.gen_loop(block, lay)[0] for l in c]
        last_read = {}
        last_bar = -1
        pending_m0 = None
        n_checked = 0
        for i, l in enumerate(lines):
            if l == "s_barrier":
                last_bar = i
                continue
            m = re.fullmatch(r"ds_read_b128 v\[\d+:\d+\], (%\[rd[AW]\]|v\d+) offset:(\d+)", l)
            if m:
                reg, off = m.group(1), int(m.group(2))
                if reg.startswith("%"):
                    op = reg[2:5]
                elif int(reg[1:]) in (g.RDA_HI, g.RDW_HI):
                    op, off = ("rdA" if int(reg[1:]) == g.RDA_HI else "rdW"), off + 65536
                else:
                    continue
                stage = ("A", off // a_bytes) if op == "rdA" else ("W", off // w_bytes)
                last_read[stage] = i
                continue
            m = re.fullmatch(r"s_add_u32 m0, %\[wave1k\], (\d+)", l)
            if m:
                pending_m0 = int(m.group(1))
                continue
            if l.startswith("buffer_load_dwordx4") and l.endswith(" lds") and "%[dSa]" not in l:
                base = pending_m0
                if base >= lay.W[0]:
                    stage = ("W", (base - lay.W[0]) // w_bytes)
                else:
                    stage = ("A", base // a_bytes)
                if stage in last_read:
                    assert last_bar > last_read[stage], (tag, block, i, l)
                    n_checked += 1
        assert n_checked > 0
