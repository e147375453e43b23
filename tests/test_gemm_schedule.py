"""CPU emulation of the MXFP4 GEMMs' stage-ring bookkeeping (k2_mx and
k2_mx8 in csrc/svdq_kernels.hip), for every K-step count 1..39 and every
low-rank chunk count 0..8 (rank up to 128).

The kernels keep a ring of LDS stages filled by global->LDS loads; each
step's loads are waited for with an immediate s_waitcnt vmcnt count, then a
workgroup barrier publishes them; a stage is refilled only after a barrier
that follows every wave's reads of its previous step.  A wrong count or a
missing request shows up here as a read of a step that is not complete, a
refill over a step still to be read, or a step never requested.  The
emulation restates the kernels' control flow step for step (waves run the
same program, so one wave's view plus barrier semantics covers all)."""
import pytest


class Ring:
    """One wave's view: load groups complete in issue order; a barrier
    publishes completed loads and finished reads to every wave."""

    def __init__(self, stages, total):
        self.S, self.total = stages, total
        self.issued = []            # steps, in issue order
        self.complete = set()       # this wave's complete load groups
        self.published = set()      # complete for every wave (after a barrier)
        self.reading = set()        # steps read, reads not yet waited for
        self.read_done = set()      # steps whose reads this wave has waited for
        self.read_published = set() # ... and every wave has (after a barrier)
        self.occupant = {}          # stage -> step
        self.reads = {}             # step -> number of reads

    def issue(self, t):
        assert 0 <= t < self.total, f"request of step {t} outside [0, {self.total})"
        assert t not in self.issued, f"step {t} requested twice"
        st = t % self.S
        prev = self.occupant.get(st)
        if prev is not None:
            assert prev in self.read_published, f"step {t} refills stage {st} before step {prev} was read by all"
        self.occupant[st] = t
        self.issued.append(t)

    def wait_vm(self, n):
        # at most n groups outstanding: all but the last n issued are complete
        for t in self.issued[:max(0, len(self.issued) - n)]:
            self.complete.add(t)

    def wait_lgkm0(self):
        self.read_done |= self.reading
        self.reading = set()

    def barrier(self):
        self.published |= self.complete
        self.read_published |= self.read_done

    def read(self, t):
        assert t in self.published, f"step {t} read before every wave's loads of it completed"
        assert self.occupant.get(t % self.S) == t, f"stage of step {t} holds step {self.occupant.get(t % self.S)}"
        self.reading.add(t)
        self.reads[t] = self.reads.get(t, 0) + 1


def emulate_k2_mx(nk, nchunks16):
    """k2_mx: 4-stage ring, the prologue requests steps 0..3, step r + 4 is
    requested into step r's own stage while step r is computed (its
    fragments were read into registers one iteration earlier); unit counts
    in load groups."""
    total = nk + (nchunks16 + 1) // 2
    R = Ring(4, total)
    for r in range(4):
        if r < total:
            R.issue(r)
    R.wait_vm(min(4, total))               # the bias (loaded before the stages) alone
    R.wait_vm(3 if total > 3 else (2 if total > 2 else (1 if total > 1 else 0)))
    R.barrier()
    R.read(0)

    def body_full(r):
        assert r + 4 < nk
        R.wait_lgkm0()
        R.wait_vm(2)
        R.barrier()
        R.read(r + 1)
        R.issue(r + 4)

    def body_tail(r):
        R.wait_lgkm0()
        if r + 1 < nk:
            R.wait_vm(int(r + 2 < total) + int(r + 3 < total))
            R.barrier()
            if r + 4 < total:
                R.issue(r + 4)
            R.read(r + 1)
        elif r + 4 < total:
            R.barrier()
            R.issue(r + 4)

    r = 0
    while r + 5 < nk:
        body_full(r)
        body_full(r + 1)
        r += 2
    while r < nk:
        body_tail(r)
        if r + 1 < nk:
            body_tail(r + 1)
        r += 2
    for q in range(nk, total):
        R.wait_lgkm0()
        R.wait_vm(0)
        R.barrier()
        R.read(q)
        if q + 4 < total:
            R.wait_lgkm0()
            R.barrier()
            R.issue(q + 4)
    return R, total


def emulate_k2_mx8(nk, nchunks16, stages):
    """k2_mx8: a STAGES-deep ring; the prologue requests STAGES steps; step
    r's stage is refilled with step r + STAGES after the phase-B barrier;
    each step is read in two halves (half 1 in phase A of its own step,
    half 0 in phase B of the step before)."""
    total = nk + (nchunks16 + 1) // 2
    R = Ring(stages, total)
    for r in range(min(stages, total)):
        R.issue(r)
    R.wait_vm(min(stages, total))          # the bias (loaded before the stages) alone
    if stages > 3 and total > 3:
        R.wait_vm(3)
    elif total > 2:
        R.wait_vm(2)
    elif total > 1:
        R.wait_vm(1)
    else:
        R.wait_vm(0)
    R.barrier()
    R.read(0)                              # step 0 half 0 and its scales

    def phase_a(r):
        R.wait_lgkm0()
        R.read(r)                          # step r half 1
        R.wait_lgkm0()

    def kstep(r):
        phase_a(r)
        R.wait_vm(stages - 2)
        R.barrier()
        R.read(r + 1)
        R.issue(r + stages)

    def kstep_tail(r):
        phase_a(r)
        if r + 1 < total:
            if stages > 3 and r + 3 < total:
                R.wait_vm(2)
            elif r + 2 < total:
                R.wait_vm(1)
            else:
                R.wait_vm(0)
            R.barrier()
        if r + stages < total:
            R.issue(r + stages)
        if r + 1 < nk:
            R.read(r + 1)

    r = 0
    while r + stages < nk:
        kstep(r)
        r += 1
    while r < nk:
        kstep_tail(r)
        r += 1
    for q in range(nk, total):
        R.wait_lgkm0()
        if q > nk:
            R.wait_vm(0)
            R.barrier()
        R.read(q)
        if q + stages < total:
            R.wait_lgkm0()
            R.barrier()
            R.issue(q + stages)
    return R, total


@pytest.mark.parametrize("nk", range(1, 40))
def test_k2_mx_stage_schedule(nk):
    for nch in range(0, 9):
        R, total = emulate_k2_mx(nk, nch)
        assert sorted(R.issued) == list(range(total)), (nk, nch)
        assert all(R.reads.get(t, 0) >= 1 for t in range(total)), (nk, nch)


@pytest.mark.parametrize("stages", [3, 4])
@pytest.mark.parametrize("nk", range(1, 40))
def test_k2_mx8_stage_schedule(nk, stages):
    for nch in range(0, 9):
        R, total = emulate_k2_mx8(nk, nch, stages)
        assert sorted(R.issued) == list(range(total)), (nk, nch, stages)
        # K steps are read in two halves, low-rank steps whole
        assert all(R.reads.get(t, 0) == (2 if t < nk else 1) for t in range(total)), (nk, nch, stages)


def test_emulation_catches_a_short_wait():
    # the emulation itself must reject a schedule with one count too large:
    # k2_mx waiting for vmcnt(3) groups in its steady step reads step r + 1
    # before it is complete
    total = 12
    R = Ring(4, total)
    for r in range(4):
        R.issue(r)
    R.wait_vm(3)
    R.barrier()
    R.read(0)
    R.wait_lgkm0()
    R.wait_vm(3)          # should be 2: it leaves steps 1, 2 and 3 in flight
    R.barrier()
    with pytest.raises(AssertionError):
        R.read(1)


def test_emulation_catches_an_early_refill():
    R = Ring(4, 12)
    for r in range(4):
        R.issue(r)
    R.wait_vm(0)
    R.barrier()
    R.read(0)             # read issued, not waited for, no barrier since
    with pytest.raises(AssertionError):
        R.issue(4)        # stage 0 refilled while step 0 is still being read


def test_emulation_catches_a_refill_without_barrier():
    # k2_mx's last K step refills its own stage: without the barrier after
    # every wave retired its reads of that step, the refill is rejected
    R = Ring(4, 12)
    for r in range(4):
        R.issue(r)
    R.wait_vm(0)
    R.barrier()
    R.read(0)
    R.wait_lgkm0()        # this wave's reads retired, not yet published
    with pytest.raises(AssertionError):
        R.issue(4)
