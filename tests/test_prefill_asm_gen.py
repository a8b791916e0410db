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
        assert lay.A[-1] + 256 * 128 <= lay.W[0] and lay.W[-1] + 32 * nw * 128 <= lay.SA[0]
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
