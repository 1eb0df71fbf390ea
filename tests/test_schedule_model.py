"""A model check of the ping-pong load bookkeeping of the tiled GEMM kernel
(schedule 2 of csrc/gemm_mfma.hpp; host-side, no GPU).

The kernel keeps loads in flight across barriers and relies on compile-time
wait counts: a wave's `s_waitcnt vmcnt(n)` retires all but its last n loads,
and the barrier that ends the phase publishes what was retired.  Two groups
of waves alternate: group g runs the load phase of slab i in barrier phase
2i + g (fragment reads of slab i, then its loads, then its wait) and the
compute phase of slab i in phase 2i + g + 1.  Every wave issues its own
share of every load, so a slab may be read in phase p only if BOTH groups
retired their shares of it in phases before p.  A load into a ring stage may
be issued in phase p only if every read of the stage's previous contents
happened in a phase before p.

The issue order and wait counts below are the kernel's (A in pairs of
slabs in a ring of 3; B in single slabs in a ring of 4, or, stored [N,K], in
pairs in a ring of 2).  The loads per wave of an A pair (A2), a B slab (B1)
and a B pair (B2) follow from each schedule-2 tile's row of the tile table
(csrc/gemm_tiles.h), and the wait counts are checked against the kernel
source's: the vmcnt expressions of its schedule-2 section must be the ones
this model evaluates.  A negative control loosens one wait count and must be
caught.
"""
import os
import re

import pytest

from parity import tile_table

KERNEL = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "activation_epilogue_gemm_amd", "csrc", "gemm_mfma.hpp")
# the schedule-2 waits of the kernel, in source order: B stored [N,K]
# prologue, B [K,N] prologue, first and second load phase of a pair with B
# pairs, the load phase with single B slabs, the drain after the loop
KERNEL_WAITS = ["A2_CH", "G::B_CH + A2_CH + G::B_CH", "A2_CH + B2_CH", "A2_CH",
                "A2_CH + 2 * G::B_CH", "0"]
SCHED2 = [t for t in tile_table() if t["sched"] == 2]


def load_counts(t):
    """(A2, B1, B2): 16-byte loads per lane of one wave for an A pair, a B
    slab and a B pair of the tile (every 64-lane load fills 1 KiB)."""
    nt = t["wm"] * t["wn"] * 64
    per = nt * 16
    return (t["bm"] * 2 * t["bk"] * 2 // per, t["bn"] * t["bk"] * 2 // per,
            t["bn"] * 2 * t["bk"] * 2 // per)


def test_model_waits_are_the_kernels():
    src = open(KERNEL).read()
    a = src.index("if constexpr (SCHED == 2) {")
    b = src.index("// prologue: the first NS-1 slabs", a)
    waits = [re.sub(r"\s+", " ", w).strip() for w in re.findall(r"wait_vmcnt<(.*?)>\(\)", src[a:b])]
    assert waits == KERNEL_WAITS, waits


def schedule(bpair: bool, npairs: int, loose: bool = False, counts=(4, 2, 4)):
    """Per-wave program: list of (kind, payload) in program order, with the
    barrier phase of each step relative to the wave's group (load phase of
    slab i is local phase 2i; the prologue is phase -1)."""
    A2, B1, B2 = counts
    prog = []
    if bpair:
        prog += [("issue", ("A", 0, 0, A2)), ("issue", ("BP", 0, 0, B2)),
                 ("issue", ("A", 1, 1, A2)), ("wait", A2), ("phase_end", -1)]
    else:
        prog += [("issue", ("A", 0, 0, A2)), ("issue", ("B", 0, 0, B1)), ("issue", ("B", 1, 1, B1)),
                 ("issue", ("A", 1, 1, A2)), ("issue", ("B", 2, 2, B1)),
                 ("wait", B1 + A2 + B1), ("phase_end", -1)]
    a_cur = 0
    for q in range(npairs):
        for h in (0, 1):
            i = 2 * q + h
            a_next = (a_cur + 2) % 3
            if bpair:
                prog.append(("read", [("A", q, a_cur), ("BP", q, q % 2)], 2 * i))
                if h == 0:
                    prog += [("issue", ("BP", q + 1, (q + 1) % 2, B2)), ("wait", A2 + B2)]
                else:
                    prog += [("issue", ("A", q + 2, a_next, A2)),
                             ("wait", A2 + (B2 if loose else 0))]
            else:
                prog.append(("read", [("A", q, a_cur), ("B", i, i % 4)], 2 * i))
                if h == 1:
                    prog.append(("issue", ("A", q + 2, a_next, A2)))
                prog += [("issue", ("B", i + 3, (i + 3) % 4, B1)),
                         ("wait", A2 + 2 * B1 - (0 if not loose else -B1))]
            prog.append(("phase_end", 2 * i))
        a_cur = (a_cur + 1) % 3
    return prog


def run_group(prog, g):
    """Global phases at which this group's share of each load retired, the
    reads it makes, and the loads it issues (with their phase)."""
    pending = []  # [(tag, count)] in issue order
    retired_at = {}
    reads, issues = [], []
    cur_local = -1
    for step in prog:
        kind = step[0]
        if kind == "issue":
            tag, num, stage, cnt = step[1]
            phase = -1 if cur_local == -1 else cur_local + g
            issues.append(((tag, num), stage, phase))
            pending.append(((tag, num), cnt))
        elif kind == "wait":
            keep = step[1]
            while sum(c for _, c in pending) > keep:
                tag, _ = pending.pop(0)
                retired_at[tag] = -1 if cur_local == -1 else cur_local + g
        elif kind == "read":
            cur_local = step[2]
            reads.append((step[1], cur_local + g))
        elif kind == "phase_end":
            pass
    return retired_at, reads, issues


def check(bpair: bool, npairs: int = 12, loose: bool = False, counts=(4, 2, 4)):
    prog = schedule(bpair, npairs, loose, counts)
    groups = [run_group(prog, g) for g in (0, 1)]
    last_slab = 2 * npairs - 1
    # readiness: every read in phase p needs both groups' shares retired before p
    for g in (0, 1):
        for needs, p in groups[g][1]:
            for tag, num, _stage in needs:
                for h in (0, 1):
                    r = groups[h][0].get((tag, num))
                    assert r is not None and r < p, (
                        f"group {g} reads {tag}{num} in phase {p}; group {h} retired it at {r}")
    # stage reuse: a load into (ring, stage) in phase p follows every read of the
    # stage's previous contents
    ring_of = {"A": "A", "BP": "B", "B": "B"}
    reads_of = {}
    for g in (0, 1):
        for needs, p in groups[g][1]:
            for tag, num, stage in needs:
                reads_of.setdefault((ring_of[tag], stage, tag, num), []).append(p)
    for g in (0, 1):
        occupant = {}
        for (tag, num), stage, p in groups[g][2]:
            key = (ring_of[tag], stage)
            prev = occupant.get(key)
            if prev is not None:
                for rp in reads_of.get((key[0], stage) + prev, []):
                    assert rp < p, f"group {g} refills {key} in phase {p}, read in {rp}"
            occupant[key] = (tag, num)
    return last_slab


@pytest.mark.parametrize("tile", SCHED2, ids=[f"tile{t['id']}" for t in SCHED2])
@pytest.mark.parametrize("bpair", [False, True])
def test_schedule2_waits_and_stage_reuse(bpair, tile):
    check(bpair, counts=load_counts(tile))


@pytest.mark.parametrize("tile", SCHED2, ids=[f"tile{t['id']}" for t in SCHED2])
@pytest.mark.parametrize("bpair", [False, True])
def test_schedule2_model_catches_a_loose_wait(bpair, tile):
    with pytest.raises(AssertionError):
        check(bpair, loose=True, counts=load_counts(tile))


def test_schedule2_tile_exists():
    assert SCHED2, "no schedule-2 tile in the tile table"
    assert load_counts(SCHED2[0]) == (4, 2, 4)
