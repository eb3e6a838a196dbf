"""CPU model of the two-group attention kernels' slot protocol (sparse_attn.hip, pingpong_attn).

The kernels stream each query tile's key blocks through per-group LDS stages, with the
LDS DMA issued from inline assembly and every wait written by hand, so nothing in the
compiler checks that a stage holds the right block when it is read.  This model replays
the protocol as the kernel source states it, slot by slot, and checks:

* every wave executes the same number of workgroup barriers (group 1 runs one slot
  behind group 0: one extra barrier at its start, group 0 one at its end);
* every read of a K or V stage in a products slot finds the block it expects, loaded
  by a DMA that was issued in an earlier slot and waited for (by the wave that issued it,
  with the kernel's own vmcnt arithmetic) before a barrier that precedes the read;
* no DMA into a stage is issued in a slot in which that stage is read, and no DMA
  replaces a stage's block before its last read;
* the V stages' zero stores complete before any DMA is issued into them (ordinary LDS
  stores and LDS DMA from different waves are not ordered by anything but a barrier).

Group G's j-th block c_j is entry 2j + G of the stream's block table; K(c_j) and V(c_j)
live in stage j % 2 of G's stages.  A products slot reads K(c_j) and V(c_{j-1}); a
softmax slot reads no stage.  The paired 64-row kernel runs one such stream per half of
each group with shared barriers, so both halves run max(n0, n1) blocks' worth of slots.
"""
import itertools

import pytest

LPK, LPT = 4, 4          # DMA loads per wave for a K and a V block (bf16, d = 128)


class ProtocolError(AssertionError):
    pass


class Stream:
    """One block stream (a query tile) and the LDS stages of its two groups."""

    def __init__(self, n):
        self.n = n
        # stage -> list of (slot issued, block label, issuing group, load ids)
        self.writes = {}
        self.reads = []          # (slot, stage, expected block label or None)

    def block(self, grp, j):
        """Table entry of group grp's j-th block, or None past the end of the list."""
        i = 2 * j + grp
        return i if 0 <= j and i < self.n else None


class Wave:
    """The vmcnt bookkeeping of one wave: its loads in issue order, and the slot by whose
    end each has landed (the kernel waits with s_waitcnt vmcnt(n): all but the newest n)."""

    def __init__(self):
        self.loads = []          # [issue slot, landed-by slot or None]

    def issue(self, slot, count):
        ids = []
        for _ in range(count):
            self.loads.append([slot, None])
            ids.append(len(self.loads) - 1)
        return ids

    def wait(self, slot, keep):
        for ld in self.loads[:max(0, len(self.loads) - keep)]:
            if ld[1] is None:
                ld[1] = slot


def run(n0, n1=None, zero_fill_before_barrier=True):
    """Replay one work item: streams of n0 (and n1 for the paired kernel) table entries.
    Returns the number of barriers each group executed."""
    streams = [Stream(n0)] + ([Stream(n1)] if n1 is not None else [])
    nmax = max(s.n for s in streams)
    iters = (nmax + 1) // 2 + 1 if nmax > 0 else 0
    waves = {(g, h): Wave() for g in (0, 1) for h in range(len(streams))}
    barriers = {0: 0, 1: 0}
    zero_slot = {}

    def dma(slot, g, h, stage, label, count):
        ids = waves[(g, h)].issue(slot, count)
        streams[h].writes.setdefault(stage, []).append((slot, label, g, ids))

    # time is counted in slots: slot t runs between the t-th and (t+1)-th workgroup barrier
    # after the block-table build; the zero stores run before that build's barrier (slot -1)
    # or, in the planted form, beside the first DMA (slot 0)
    zslot = -1 if zero_fill_before_barrier else 0
    for h, s in enumerate(streams):
        for g in (0, 1):
            for st in (0, 1):
                zero_slot[(h, ("V", g, st))] = zslot

    # prologue (slot 0): K(c_0), K(c_1), V(c_0) of the group's own stream, then
    # wait_vm(np), barrier; group 1 then takes one more barrier (slot 1 idle)
    np_ = {}
    for g in (0, 1):
        for h, s in enumerate(streams):
            c0, c1 = s.block(g, 0), s.block(g, 1)
            if c0 is not None:
                dma(0, g, h, ("K", g, 0), ("K", c0), LPK)
            if c1 is not None:
                dma(0, g, h, ("K", g, 1), ("K", c1), LPK)
            n = 0
            if c0 is not None:
                dma(0, g, h, ("V", g, 0), ("V", c0), LPT)
                n = LPT
            waves[(g, h)].wait(0, n)
            np_[(g, h)] = n if g == 0 else 0
        barriers[g] += 1
    barriers[1] += 1

    # group 0 runs phase p in slot p + 1, group 1 in slot p + 2; phase 2j is the products
    # slot of c_j, phase 2j + 1 its softmax slot
    xo = {(g, h): (streams[h].block(0, 1) if g == 1 else None) for g in (0, 1) for h in range(len(streams))}
    for p in range(2 * iters):
        j, products = p // 2, p % 2 == 0
        st = j % 2
        for g in (0, 1):
            slot = p + 1 + g
            for h, s in enumerate(streams):
                w = waves[(g, h)]
                if products:
                    cj, cjm1 = s.block(g, j), s.block(g, j - 1)
                    s.reads.append((slot, ("K", g, st), ("K", cj) if cj is not None else None))
                    s.reads.append((slot, ("V", g, 1 - st), ("V", cjm1) if cjm1 is not None else None))
                    nc = 0
                    if xo[(g, h)] is not None:
                        # group 1 fills group 0's V stage (j+1)%2, group 0 fills group 1's V stage j%2
                        tgt = ("V", 1 - g, (1 - st) if g == 1 else st)
                        dma(slot, g, h, tgt, ("V", xo[(g, h)]), LPT)
                        nc = LPT
                else:
                    nc = 0
                    cj2 = s.block(g, j + 2)
                    if cj2 is not None:
                        dma(slot, g, h, ("K", g, st), ("K", cj2), LPK)
                        nc = LPK
                    # the other group's block whose V the next products slot loads
                    io = 2 * (j + 2) if g == 1 else 2 * (j + 1) + 1
                    xo[(g, h)] = io if io < s.n else None
                w.wait(slot, nc + np_[(g, h)])
                np_[(g, h)] = nc
            barriers[g] += 1
    barriers[0] += 1                                  # group 0 matches group 1's first slot
    for w in waves.values():
        w.wait(10 ** 9, 0)                            # vmcnt(0) before the merge

    # checks
    for h, s in enumerate(streams):
        for slot, stage, want in s.reads:
            before = [wr for wr in s.writes.get(stage, []) if wr[0] < slot]
            same = [wr for wr in s.writes.get(stage, []) if wr[0] == slot]
            if same:
                raise ProtocolError(f"stream {h}: {stage} read in slot {slot} while a DMA into it is issued there")
            if want is None:
                continue                              # a missing block: P = 0, any finite contents
            if not before or before[-1][1] != want:
                got = before[-1][1] if before else "zero fill"
                raise ProtocolError(f"stream {h}: slot {slot} reads {stage} expecting {want}, holds {got}")
            wslot, _, g, ids = before[-1]
            for i in ids:
                landed = waves[(g, h)].loads[i][1]
                if landed is None or landed >= slot:
                    raise ProtocolError(f"stream {h}: slot {slot} reads {stage} ({want}) before its DMA "
                                        f"(issued in slot {wslot}) was waited for")
        for stage, wrs in s.writes.items():
            z = zero_slot.get((h, stage))
            if z is not None and any(wr[0] <= z for wr in wrs):
                raise ProtocolError(f"stream {h}: DMA into {stage} in the slot of its zero stores")
    if barriers[0] != barriers[1]:
        raise ProtocolError(f"barrier counts differ: {barriers}")
    return barriers[0]


@pytest.mark.parametrize("n", range(0, 80))
def test_two_group_stream(n):
    """128-row kernels: one stream of n table entries (every block count up to 79)."""
    b = run(n)
    assert b == (2 + 2 * ((n + 1) // 2 + 1) if n > 0 else 2)


def test_paired_streams():
    """Paired 64-row kernel: two streams of different lengths share the barriers; the
    shorter one runs its extra slots on missing blocks."""
    for n0, n1 in itertools.product(range(0, 24), repeat=2):
        run(n0, n1)
    for n0, n1 in [(60, 3), (3, 60), (61, 60), (79, 0), (0, 79)]:
        run(n0, n1)


def test_zero_stores_beside_the_first_dma_are_flagged():
    """The earlier ordering (V stages zeroed next to the first DMA, after the barrier) is a
    race between one wave's zero stores and another wave's DMA; the model reports it."""
    with pytest.raises(ProtocolError, match="zero stores"):
        run(5, zero_fill_before_barrier=False)
    run(5)


def test_model_catches_a_missing_wait():
    """A planted off-by-one in the wait arithmetic (waiting for one phase less) is caught."""
    orig = Wave.wait

    def lax(self, slot, keep):
        return orig(self, slot, keep + LPT)
    Wave.wait = lax
    try:
        with pytest.raises(ProtocolError, match="before its DMA"):
            for n in range(1, 12):
                run(n)
    finally:
        Wave.wait = orig
