"""The counted waits of the persistent weight-gradient loop (host model).

The weight-gradient kernel waits for a K-step's direct-to-LDS loads with
s_waitcnt vmcnt(n): at most n vector memory operations of the wave may still
be outstanding, and they complete in issue order, so the wait holds exactly
when fewer than n + 1 operations were issued after the K-step's loads.  Its
ring of NS = 4 stages issues K-step kt + 3 during K-step kt (NQ = 4 loads per
wave: two 1 KB pieces of each 256 x 32 operand tile), the first PRE = 2
K-steps of a tile are issued before the previous tile's epilogue, and the
epilogue's operations then drain under the first K-steps:
  - bf16 output: 16 stores per wave (two column halves of 8), waits
    vmcnt(2 NQ + 16) at K-steps 0 and 1;
  - fp32 accumulate-into: 32 loads and 32 stores per wave in four passes (the
    loads of a pass before its stores), waits vmcnt(2 NQ + 8) there;
  - later K-steps wait vmcnt(2 NQ).
Replaying the issue order of a run of tiles, every wait must leave the
K-step's own loads outside the allowed count, whatever the tiles' K-step
counts (an empty expert issues nothing; a one-K-step tile still issues its
second prefetched K-step and the ring's zero loads past K).
"""
import pytest

NQ, NS, PRE = 4, 4, 2


def epilogue_ops(f32):
    if f32:
        ops = []
        for _ in range(4):
            ops += ["cload"] * 8 + ["cstore"] * 8
        return ops
    return ["store"] * 16


def replay(nks, f32, ndrain=None):
    """Issue order of the wave's vector memory operations over tiles with the
    given K-step counts; returns (log, waits) where waits holds (position of
    the wait, the K-step load tag it needs, allowed outstanding count)."""
    if ndrain is None:
        ndrain = 8 if f32 else 16
    log, waits = [], []

    def issue(tag, n=NQ):
        log.extend([tag] * n)

    # first tile: its first PRE K-steps, no epilogue before them
    if nks[0] > 0:
        for j in range(PRE):
            issue(("L", 0, j))
    stores_drain = False
    for t, nk in enumerate(nks):
        if nk > 0:
            for j in range(PRE, NS - 1):                # prologue of the ring
                issue(("L", t, j))
            for kt in range(nk):
                allow = 2 * NQ + (ndrain if stores_drain and kt < PRE else 0)
                waits.append((len(log), ("L", t, kt), allow))
                issue(("L", t, kt + NS - 1))            # loads NS - 1 K-steps ahead (zeros past K)
        # next tile's first PRE K-steps, then this tile's epilogue
        if t + 1 < len(nks) and nks[t + 1] > 0:
            for j in range(PRE):
                issue(("L", t + 1, j))
        log.extend(epilogue_ops(f32))
        stores_drain = True
    return log, waits


def check(nks, f32, ndrain=None):
    log, waits = replay(nks, f32, ndrain)
    for pos, tag, allow in waits:
        last = max(i for i in range(pos) if log[i] == tag)     # the K-step's last load issued
        after = pos - 1 - last                                    # operations issued after it
        assert after >= allow, (nks, f32, tag, after, allow)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("nks", [[16, 16, 16], [1, 1, 1], [16, 0, 16], [0, 5, 0, 1, 2], [2, 3, 1, 16, 1],
                                 [1], [256, 1, 256]])
def test_waits_never_allow_the_needed_loads(nks, f32):
    check(nks, f32)


@pytest.mark.parametrize("f32,tight", [(False, 16), (True, 64)])
def test_the_drain_counts_are_exact_or_safe(f32, tight):
    # the bf16 allowance is exact (one more would let K-step 0's loads be
    # outstanding); the fp32 one (8) is below the 64 its epilogue leaves room for
    check([16, 16, 16], f32, tight)
    with pytest.raises(AssertionError):
        check([16, 16, 16], f32, tight + 1)
