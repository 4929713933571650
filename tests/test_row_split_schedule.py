"""Host check of the row-split GEMM's compile-time load schedule (the loop of
csrc/gemm_ns.h), written out in Python from its description there.

A wave walks passes of ng groups of R ring slots, K block by K block, tile by
tile; at each step it waits with vmcnt(W), reads the visit from its slot,
refills that slot with the visit R steps ahead and multiplies; every block
start waits, passes a barrier and issues the next block's A-staging loads.
Loads retire in issue order, so after `s_waitcnt vmcnt(W)` every load except
the W most recent has landed.  The simulation issues the loads in the kernel's
order and asserts, for every shape the kernel is built for (every row-tile
count and ring depth, one to three passes, one to four K blocks, every group
count):
  * at each step, the visit being read has landed (at least W loads were
    issued after it) and W is exactly that count (the waits are not stricter
    than they need to be);
  * at each block start, that block's A-staging loads have landed;
  * every slot holds the visit its step expects (the right tile, K block and
    pass), so no refill overwrites a slot before it is read;
  * every tile of every pass is multiplied once per K block."""
import itertools

import pytest

from gpu_util import NTW_MAX, RINGS

# loads per visit (bf16: 16 rows x 256 bytes in 1 KB loads; fp8: 128 bytes)
NI = {"bf16": 4, "fp8": 2}


def kernel_step_wait(ni, na, R, T):
    """vmcnt of step T: R - 1 visits followed visit T, and the block's A
    loads too while T < R."""
    return ni * (R - 1) + (na if T < R else 0)


def kernel_block_wait(ni, R):
    """vmcnt at a block start: at least R visits followed its A loads."""
    return ni * R


def simulate(ni, na, R, ng, npass, nblk, step_wait=kernel_step_wait,
             block_wait=kernel_block_wait):
    """Run the schedule; returns the number of visits multiplied."""
    issued = []          # load tags in issue order
    slot = {}            # ring slot -> visit tag it holds
    pos_of = {}          # visit tag -> index of its last load in `issued`

    def issue_visit(tag, s):
        for _ in range(ni):
            issued.append(tag)
        pos_of[tag] = len(issued) - 1
        slot[s] = tag

    def issue_a(tag):
        for _ in range(na):
            issued.append(tag)
        pos_of[tag] = len(issued) - 1

    def after(tag):      # loads issued after the last load of `tag`
        return len(issued) - 1 - pos_of[tag]

    tiles = ng * R
    blocks = [(p, kb) for p in range(npass) for kb in range(nblk)]

    def visit_tag(bi, t):
        if bi >= len(blocks):
            return ("oob", bi, t)
        p, kb = blocks[bi]
        return ("w", p, kb, t)

    # prologue: A of the first block, then tiles 0 .. R - 1 of pass 0
    issue_a(("a", 0))
    for t in range(R):
        issue_visit(visit_tag(0, t), t)
    done = 0
    for bi in range(len(blocks)):
        # block start: this block's A slice landed, barrier, next block's A
        assert after(("a", bi)) >= block_wait(ni, R), ("A slice not landed", bi)
        issue_a(("a", bi + 1))
        for G in range(ng):
            last_g = G + 1 >= ng
            for J in range(R):
                T = G * R + J
                want = visit_tag(bi, T)
                w = step_wait(ni, na, R, T)
                assert slot[J] == want, ("wrong visit in slot", bi, T, slot[J], want)
                assert after(want) >= w, ("visit not landed", bi, T, after(want), w)
                assert after(want) == w, ("wait stricter than needed", bi, T, after(want), w)
                # reads done: refill this slot with the visit R steps ahead
                nxt = visit_tag(bi + 1, J) if last_g else visit_tag(bi, (G + 1) * R + J)
                issue_visit(nxt, J)
                done += 1
        assert done == (bi + 1) * tiles
    return done


CASES = [(mt, R) for mt, rs in RINGS.items() for R in rs]


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("mt,R", CASES)
def test_schedule_waits_and_slots(weights, mt, R):
    ni = NI[weights]
    ng_max = NTW_MAX[mt] // R
    assert ng_max >= 1
    assert ni * (R - 1) + mt <= 63        # vmcnt range of the kernel's waits
    for ng, npass, nblk in itertools.product(range(1, ng_max + 1), (1, 2, 3), (1, 2, 4)):
        n = simulate(ni, mt, R, ng, npass, nblk)
        assert n == ng * R * npass * nblk


@pytest.mark.parametrize("step_wait", [
    lambda ni, na, R, T: ni * (R - 1),                          # A loads left out
    lambda ni, na, R, T: ni * (R - 1) + na + 1,                 # one load too loose
    lambda ni, na, R, T: ni * R + (na if T < R else 0),         # one visit too loose
])
def test_simulation_rejects_wrong_waits(step_wait):
    """The simulation is sensitive: step waits that leave out the A loads or
    allow one load or one visit too many in flight fail it."""
    with pytest.raises(AssertionError):
        simulate(4, 8, 5, 2, 2, 2, step_wait=step_wait)


def test_simulation_rejects_a_looser_block_wait():
    """A block-start wait that allows more loads in flight than followed the
    block's A slice fails it."""
    with pytest.raises(AssertionError):
        simulate(4, 8, 5, 1, 1, 2, block_wait=lambda ni, R: ni * R + ni * R + 9)
