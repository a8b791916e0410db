"""LDS races of the generated prefill K loop, checked on the CPU.

Every wave of a workgroup runs the same instruction stream (waves 0 .. tm/64 - 1
also copy the activation scales; the others branch around those copies), and
the waves meet only at s_barrier.  So a data race on LDS shows up in one
wave's stream read against the counter rules of the hardware:

- vector-memory operations (the copies into LDS, `buffer_load ... lds`)
  complete in issue order; `s_waitcnt vmcnt(n)` returns when at most the last
  n issued are still outstanding;
- LDS operations (`ds_read*`) likewise under `s_waitcnt lgkmcnt(n)`;
- another wave's operation is known complete only if it completed before a
  barrier that this wave has since passed.

The checker interprets the stream of each (shape, scale mode) for several K
lengths, follows its branches (the K-loop exits and the scale-copy waves),
tracks which LDS region (an operand stage, an activation-scale group buffer,
the weight-scale table) every copy writes and every read reads, and asserts

- read after write: a read of a region comes after a barrier that followed
  the completion of every copy into that region issued before it;
- write after read: a copy into a region comes after a barrier that followed
  the completion of every read of that region issued before it;
- the epilogue's barrier finds nothing outstanding (its staging area
  overlaps the stages).

Mistakes planted into the stream (a barrier's wait one copy short, a missing
LDS wait before a barrier, a copy moved ahead of its barrier) are caught."""
import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "fp8_w8a8_block_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_prefill_asm",
                                                  os.path.join(CSRC, "gen_prefill_asm.py"))
    g = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(g)
    return g


G = _gen()


class Race(AssertionError):
    pass


def _regions(lay):
    a_bytes, w_bytes = lay.a_units * lay.unit, lay.w_units * lay.unit
    group = lay.SA[1] - lay.SA[0]

    def copy_region(m0):
        kind, off = m0
        if kind == "wave1k":
            if off >= lay.W[0]:
                s = (off - lay.W[0]) // w_bytes
                assert s < len(lay.W)
                return ("W", s)
            s = off // a_bytes
            assert s < len(lay.A)
            return ("A", s)
        if kind == "sam0":
            assert off % group == 0 and off // group in (0, 1)
            return ("SA", off // group)
        assert kind == "swm0"
        return ("SW", 0)

    def read_region(l):
        m = re.fullmatch(r"ds_read_b128 v\[\d+:\d+\], (%\[rd[AW]\]|v\d+) offset:(\d+)", l)
        if m:
            reg, off = m.group(1), int(m.group(2))
            if reg.startswith("%"):
                op = reg[2:5]
            else:
                r = int(reg[1:])
                assert r in (G.RDA_HI, G.RDW_HI), l
                op, off = ("rdA" if r == G.RDA_HI else "rdW"), off + 65536
            return ("A", off // a_bytes) if op == "rdA" else ("W", off // w_bytes)
        m = re.fullmatch(r"ds_read2_b32 v\[\d+:\d+\], %\[sc[LH]([01])\] offset0:\d+ offset1:\d+", l)
        if m:
            return ("SA", int(m.group(1)))
        if re.fullmatch(r"ds_read_b32 v\d+, %\[swrd\]", l):
            return ("SW", 0)
        raise AssertionError(f"unexpected LDS operation in the K loop: {l}")

    return copy_region, read_region


def simulate(lines, lay, KB, wsa, split=False):
    """Interpret one wave's stream up to the epilogue's barrier; raise Race on
    a violation.  split: a split-K launch, whose waves first record their XCD
    (one store, counted by the same counter as the copies).  Returns the
    number of steps run and of reads checked."""
    copy_region, read_region = _regions(lay)
    labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}
    vm, lgkm = [], []              # outstanding operations, issue order
    copies, reads = {}, {}         # region -> [op] (op: dict with 'done' epoch)
    epoch = 0                      # barriers passed
    skb, scc, m0 = None, None, None
    tail_seen, steps, checked = False, 0, 0
    pc = 0
    while True:
        assert pc < len(lines), "ran off the end of the stream"
        l = lines[pc]
        pc += 1
        if l.endswith(":"):
            if l.startswith("fp8pf_tail_"):
                tail_seen = True
            continue
        if l == "s_barrier":
            if tail_seen:
                if vm or lgkm:
                    raise Race(f"epilogue barrier with {len(vm)} copies and {len(lgkm)} "
                               f"LDS operations outstanding")
                return steps, checked
            epoch += 1
            continue
        m = re.fullmatch(r"s_waitcnt(?: vmcnt\((\d+)\))?(?: lgkmcnt\((\d+)\))?", l)
        if m:
            for q, n in ((vm, m.group(1)), (lgkm, m.group(2))):
                if n is not None:
                    while len(q) > int(n):
                        q.pop(0)["done"] = epoch
            continue
        # scalar control: the K counter, the loop's exits, the scale-copy waves
        if l == "s_mov_b32 s84, 0":
            skb = 0
            continue
        if l == "s_add_u32 s84, s84, 1":
            skb += 1
            steps += 1
            continue
        if l.startswith("s_cmp"):
            if l == "s_cmp_eq_u32 s84, %[kb]":
                scc = skb == KB
            elif l == "s_cmp_lt_u32 s84, %[kb]":
                scc = skb < KB
            elif l == "s_cmp_eq_u32 %[wsa], 0":
                scc = wsa == 0
            elif l == "s_cmp_eq_u32 %[xinfo], 0":
                scc = not split
            elif l == "s_cmp_eq_u32 %[colok], 0":
                scc = False
            else:
                raise AssertionError(f"unexpected compare before the epilogue: {l}")
            continue
        m = re.fullmatch(r"s_cbranch_scc([01]) (\S+)", l)
        if m:
            if scc == (m.group(1) == "1"):
                pc = labels[m.group(2)]
            continue
        # copies into LDS and the m0 that places them
        m = re.fullmatch(r"s_add_u32 m0, %\[(wave1k|sam0)\], (\d+)", l)
        if m:
            m0 = (m.group(1), int(m.group(2)))
            continue
        if l == "s_mov_b32 m0, %[swm0]":
            m0 = ("swm0", 0)
            continue
        if l.startswith("buffer_load") and l.endswith(" lds"):
            reg = copy_region(m0)
            # write after read: every earlier read of the region completed
            # before a barrier this wave has passed
            for r in reads.get(reg, []):
                if r["done"] is None or r["done"] >= epoch:
                    raise Race(f"copy into {reg} at step {skb} before every wave's read of it "
                               f"is known complete: {l}")
            op = {"done": None}
            vm.append(op)
            copies.setdefault(reg, []).append(op)
            continue
        if split and l.startswith("buffer_store_dword ") and "%[dWs]" in l:
            vm.append({"done": None})  # the XCD record: no LDS region
            continue
        if l.startswith("buffer_") or l.startswith("s_sleep"):
            raise AssertionError(f"unexpected memory operation before the epilogue: {l}")
        if l.startswith("ds_"):
            reg = read_region(l)
            for c in copies.get(reg, []):
                if c["done"] is None or c["done"] >= epoch:
                    raise Race(f"read of {reg} at step {skb} before every wave's copy into it "
                               f"is known complete: {l}")
            op = {"done": None}
            lgkm.append(op)
            reads.setdefault(reg, []).append(op)
            checked += 1
            continue
        # everything else (VALU, MFMA, SALU address arithmetic) touches no LDS


def _cases():
    return [(tag, block) for tag in G.SHAPES for block in (True, False)]


def _kbs(lay):
    # K lengths: the shortest, each exit of the unrolled loop, one and a
    # half periods, and a long one
    P = G.loop_period(lay.stages)
    return sorted({4, 8, 12, P, P + 4, P + P // 2, 4 * P + 4})


@pytest.mark.parametrize("tag,block", _cases())
def test_generated_loop_has_no_lds_race(tag, block):
    lay = G.layout(tag)
    lines, _ = G.gen(block, tag)
    for KB in _kbs(lay):
        for wsa in (0, 1):
            for split in ((False, True) if tag == G.SPLIT_SHAPE else (False,)):
                steps, checked = simulate(lines, lay, KB, wsa, split)
                assert steps == KB, (tag, block, KB, wsa, split)
                assert checked > 0


def _loop_slice(lines):
    lo = next(i for i, l in enumerate(lines) if l.startswith("fp8pf_loop_"))
    hi = next(i for i, l in enumerate(lines) if l.startswith("fp8pf_tail_"))
    return lo, hi


def _first_loop_barrier(lines):
    lo, hi = _loop_slice(lines)
    return next(i for i in range(lo, hi) if lines[i] == "s_barrier")


def _expect_race(lines, lay):
    with pytest.raises(Race):
        for KB in _kbs(lay):
            for wsa in (0, 1):
                simulate(lines, lay, KB, wsa)


@pytest.mark.parametrize("tag,block", _cases())
def test_a_short_copy_wait_is_caught(tag, block):
    # the barrier's copy wait leaves one more copy outstanding: the next
    # step reads a stage whose last copy may still be landing
    lay = G.layout(tag)
    lines, _ = G.gen(block, tag)
    b = _first_loop_barrier(lines)
    i = max(j for j in range(b) if lines[j].startswith("s_waitcnt vmcnt("))
    n = int(re.search(r"vmcnt\((\d+)\)", lines[i]).group(1))
    bad = list(lines)
    bad[i] = lines[i].replace(f"vmcnt({n})", f"vmcnt({n + 1})")
    _expect_race(bad, lay)


@pytest.mark.parametrize("tag,block", _cases())
def test_a_missing_lds_wait_before_a_barrier_is_caught(tag, block):
    # without the LDS wait the wave's reads of the stage may still be in
    # flight when the copies after the barrier overwrite it
    lay = G.layout(tag)
    lines, _ = G.gen(block, tag)
    b = _first_loop_barrier(lines)
    i = max(j for j in range(b) if lines[j] == "s_waitcnt lgkmcnt(0)")
    assert b - i <= 2
    bad = lines[:i] + lines[i + 1:]
    _expect_race(bad, lay)


@pytest.mark.parametrize("tag,block", _cases())
def test_a_copy_ahead_of_its_barrier_is_caught(tag, block):
    # the step's first copy moved above its barrier overwrites a stage that
    # other waves may still be reading
    lay = G.layout(tag)
    lines, _ = G.gen(block, tag)
    lo, hi = _loop_slice(lines)
    b = _first_loop_barrier(lines)
    c = next(i for i in range(b, hi) if lines[i].startswith("buffer_load") and
             lines[i].endswith(" lds") and "%[dSa]" not in lines[i])
    m = max(j for j in range(b, c) if lines[j].startswith("s_add_u32 m0"))
    assert lines[m + 1] == "s_nop 0" and c == m + 2
    w = b
    while lines[w - 1].startswith("s_waitcnt"):
        w -= 1
    moved = [lines[m], "s_nop 0", lines[c]]
    bad = lines[:w] + moved + [l for k, l in enumerate(lines[w:], w) if k not in (m, m + 1, c)]
    _expect_race(bad, lay)
