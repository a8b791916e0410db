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


def test_fixed_registers_and_lds_fit():
    g = _gen()
    assert g.NUM_FIXED_VGPR + 11 <= 256          # fixed map plus the C++ operands
    for nw in g.SHAPES:
        lay = g.Layout(nw, g.STAGES[nw])
        assert lay.bytes <= 160 * 1024
        # stages, then the scale groups and the table, none overlapping
        assert lay.A[-1] + 32 * lay.unit <= lay.W[0] and lay.W[-1] + 4 * nw * lay.unit <= lay.SA[0]
    for nw, block in [(nw, b) for nw in g.SHAPES for b in (True, False)]:
        lines, max_out = g.gen(block, nw)
        assert max_out <= 15
        regs = [int(m) for l in lines for m in re.findall(r"\bv(\d+)\b", l)]
        regs += [int(b) for l in lines for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", l)]
        assert max(regs) < g.NUM_FIXED_VGPR


def test_every_lds_wait_names_a_smaller_count():
    # counts in s_waitcnt lgkmcnt(n) stay encodable (4 bits)
    g = _gen()
    for nw, block in [(nw, b) for nw in g.SHAPES for b in (True, False)]:
        lines, _ = g.gen(block, nw)
        for l in lines:
            m = re.match(r"s_waitcnt lgkmcnt\((\d+)\)", l)
            if m:
                assert int(m.group(1)) <= 15


def test_barriers_wait_for_the_next_block():
    # with S stages, the copies a step issues are for block kb + S and its
    # barrier must leave at most the copies issued after block kb + 1 in
    # flight: 8 per step for 256 x 256 tiles with two stages (so none), 12 per
    # step for 256 x 128 tiles with three (plus at most one scale copy)
    g = _gen()
    for nw, block in [(nw, b) for nw in g.SHAPES for b in (True, False)]:
        lines, _ = g.gen(block, nw)
        # the waits right before a barrier: the prologue's, then one per step
        waits = [int(m.group(1)) for l, nxt in zip(lines, lines[1:]) if nxt == "s_barrier"
                 for m in [re.fullmatch(r"s_waitcnt vmcnt\((\d+)\)", l)] if m]
        n = len(g.copies(nw))
        loop = waits[1:]
        assert len(loop) == g.loop_period(g.STAGES[nw])
        if g.STAGES[nw] == 2:
            assert set(loop) == {0}
        else:
            assert set(loop) <= {n, n + 1} and waits[0] == (g.STAGES[nw] - 1) * n


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

    for nw in g.SHAPES:
        lay = g.Layout(nw, g.STAGES[nw])
        for j in range(8):                                   # fragment of the wave
            for half in range(2):                            # first or second ds_read_b128
                for kg in range(4):                          # 16-lane group
                    addrs = []
                    for r16 in range(16):
                        row = 16 * j + r16
                        pos = (2 * kg) ^ swz_pair(r16)
                        addrs.append((row // 8) * lay.unit + (row % 8) * 128 + pos * 16 + 16 * half)
                    assert len(set(_bank_groups(addrs))) == 16, (nw, j, half, kg)
        # the unpadded layout meets every bank twice
        flat = g.Layout(nw, g.STAGES[nw], pad=0)
        addrs = [(r // 8) * flat.unit + (r % 8) * 128 + swz_pair(r) * 16 for r in range(16)]
        assert len(set(_bank_groups(addrs))) == 8


def test_copies_land_where_fragments_are_read():
    # copy t of wave w writes tile rows 8 (w + NW t) .. + 7 as one 1 KiB unit
    # at stage + (w + NW t) * unit; fragment j of wave row wm starts at unit
    # 16 wm + 2 j: the two addressings agree for every row
    g = _gen()
    for nw in g.SHAPES:
        lay = g.Layout(nw, g.STAGES[nw])
        seen = set()
        for w in range(nw):
            for t in range(32 // nw):
                u = w + nw * t
                for r in range(8):
                    row = 8 * u + r
                    wm, j, r16 = row // 128, (row % 128) // 16, row % 16
                    by_read = wm * 16 * lay.unit + j * lay.frag + (r16 // 8) * lay.unit + (r16 % 8) * 128
                    by_copy = u * lay.unit + r * 128
                    assert by_read == by_copy
                    seen.add(row)
        assert seen == set(range(256))
        assert lay.A[1] - lay.A[0] == 32 * lay.unit and lay.W[0] == lay.stages * 32 * lay.unit


def test_split_handover_stays_in_its_slot():
    # every workspace access of the split-K hand-over lies inside the wave's
    # slot: its four words (16 bytes at 16 slot) and its 32 KiB partial (quad
    # q of lane l at 1024 q + 16 l); the 256 x 128 shape has no hand-over
    g = _gen()
    for block in (True, False):
        lines, _ = g.gen(block, 8)
        base = None
        seen = 0
        for l, nxt in zip(lines, lines[1:] + [""]):
            m = re.fullmatch(r"s_add_u32 s88, %\[wsPart\], (\d+)", l)
            if m:
                base = int(m.group(1))
                assert base % 4096 == 0 and base < g.SPLIT_PART_BYTES
            if l == f"s_sub_u32 s88, %[wsPart], {g.SPLIT_WORDS_BYTES}":
                assert nxt == "s_lshr_b32 s88, s88, 11"      # 16 bytes per 32 KiB slot
                base = "words"
            if "%[dWs]" in l:
                seen += 1
                off = int(re.search(r"offset:(\d+)", l).group(1)) if "offset:" in l else 0
                assert "s88" in l and base is not None
                if base == "words":                          # the words (voffset 0 or 8 / 12)
                    assert off in (0, 4)
                else:                                        # a 16-byte quad, lane offset <= 1008
                    assert l.startswith(("buffer_load_dwordx4", "buffer_store_dwordx4"))
                    assert base + off + 1008 + 16 <= g.SPLIT_PART_BYTES
        assert seen == 1 + 1 + 1 + 2 * 32 + 1 + 1 + 2 * 32      # record, atomic, partner, stores, flag, poll, loads
        for l in g.gen(block, 4)[0]:
            assert "%[dWs]" not in l
