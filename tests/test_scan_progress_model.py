"""Forward progress of the persistent scan, checked on a model of its workgroups (CPU only).

The model follows the kernel's schedule per workgroup: workgroup b, of group g = b mod 8, takes
a rank r in its group as it starts and claims tiles from counter (g + r) mod nc while r < nc,
else from counter g mod nc (the k-th claim of counter c is tile k * nc + c); a tile's local
step publishes its
total and, for the last tile of an anchor interval, waits for the interval's tile totals and
publishes the interval total; the last tile of a super-interval also waits for the
super-interval's interval totals and the previous carry and publishes the next carry; a tile's
finish waits for the earlier tile totals of its interval, the earlier interval totals of its
super-interval and its carry.  Per workgroup: claim c, local(c), then repeatedly local(u),
take the ticket claimed earlier as v and claim the next, finish(c), shift.  Random
interleavings of workgroup steps must always finish.  With the carry forwarded from the
finish of the super-interval's last tile instead (the schedule the kernel once had), the
model finds the cycle: that finish waits behind the workgroup's next local step, which can
close a later interval whose tiles' workgroups wait for the carry.

Grids larger than the number of workgroups that fit at once (a test hook of the library) are
modelled by a dispatch queue: workgroups start in index order, at most `resident` at a time,
and a waiting one starts only when a running one has returned.  The host uses no more claim
counters than resident workgroups; with more, a counter can be left with no running workgroup
while the running ones wait on its tiles, and the model finds that stall.

Two scans sharing the chip (two streams) are modelled with per-XCD slots: workgroup b of a grid
goes to XCD b mod 8 and each XCD starts its share of a grid in index order, taking the grids'
queued workgroups in a random mix.  With the counter tied to the workgroup index (b mod nc, the
kernel's earlier choice) the model finds interleavings where each scan holds every slot of an
XCD that the other needs for one of its counters, and both wait forever; by start rank every
interleaving finishes as long as an XCD has nc slots per scan (a scan one of whose groups has
started nc workgroups proceeds; an MI355X XCD has 64 or more per scan kernel).  With fewer (one
slot per XCD, two scans) both can stop short, which the model also shows.
"""
import random

import pytest


class Model:
    def __init__(self, ntiles, A, A2, nwg, carry_in_local, seed, resident=None, by_rank=True):
        self.N, self.A, self.A2 = ntiles, A, A2
        self.resident = nwg if resident is None else min(resident, nwg)
        self.nc = min(8, nwg, self.resident)      # the host never uses more counters
        self.ctr = [0] * self.nc
        self.by_rank = by_rank
        self.ranks = [0] * 8                      # workgroups started so far, per group
        self.wg_ctr = {}                          # workgroup -> its counter
        self.agg, self.G, self.carry = set(), set(), {0}   # carry[0]: the identity, always known
        self.local_carry = carry_in_local
        self.rng = random.Random(seed)
        self.wgs = [self.program(b) for b in range(nwg)]
        self.pending = [next(w) for w in self.wgs]          # each yields (wait-set, action)

    def claim(self, b):
        if b not in self.wg_ctr:                  # first claim: the counter from the start rank
            g = b % 8
            r = self.ranks[g]
            self.ranks[g] += 1
            if self.by_rank:
                self.wg_ctr[b] = (g + r) % self.nc if r < self.nc else g % self.nc
            else:
                self.wg_ctr[b] = b % self.nc
        c = self.wg_ctr[b]
        t = self.ctr[c] * self.nc + c
        self.ctr[c] += 1
        return t

    def lb(self, t):
        q = t // self.A
        return q, t - q * self.A, q // self.A2, q - (q // self.A2) * self.A2

    def local(self, t):
        # publish the tile total, then (anchors) the interval total and (super-interval
        # anchors, with the carry forwarded here) the next carry
        yield (set(), lambda: self.agg.add(t))
        q, cnt, Q, qcnt = self.lb(t)
        if cnt == self.A - 1 and t + 1 < self.N:
            need = {("a", q * self.A + i) for i in range(cnt)}
            yield (need, lambda: self.G.add(q))
            if self.local_carry and qcnt == self.A2 - 1:
                need = {("g", Q * self.A2 + i) for i in range(qcnt)} | {("c", Q)}
                yield (need, lambda: self.carry.add(Q + 1))

    def finish(self, t):
        q, cnt, Q, qcnt = self.lb(t)
        need = ({("a", q * self.A + i) for i in range(cnt)}
                | {("g", Q * self.A2 + i) for i in range(qcnt)} | {("c", Q)})
        sanchor = cnt == self.A - 1 and t + 1 < self.N and qcnt == self.A2 - 1
        if sanchor and not self.local_carry:
            yield (need, lambda: self.carry.add(Q + 1))
        else:
            yield (need, lambda: None)

    def program(self, b):
        box = {}
        yield (set(), lambda: box.__setitem__("c", self.claim(b)))
        c = box["c"]
        if c >= self.N:
            return
        yield (set(), lambda: box.__setitem__("k", self.claim(b)))
        yield from self.local(c)
        u = box["k"]
        if u < self.N:
            yield (set(), lambda: box.__setitem__("k", self.claim(b)))
        while True:
            if u < self.N:
                yield from self.local(u)
            v = box["k"] if u < self.N else self.N
            if v < self.N:
                yield (set(), lambda: box.__setitem__("k", self.claim(b)))
            yield from self.finish(c)
            if u >= self.N:
                return
            c, u = u, v

    def ready(self, need):
        for kind, i in need:
            if kind == "a" and i not in self.agg:
                return False
            if kind == "g" and i not in self.G:
                return False
            if kind == "c" and i not in self.carry:
                return False
        return True

    def run(self):
        """True if every workgroup finishes; False at the first state where none can move."""
        nwg = len(self.wgs)
        live = list(range(self.resident))        # dispatched in index order
        queued = self.resident                    # next workgroup waiting for a slot
        while live:
            movable = [b for b in live if self.ready(self.pending[b][0])]
            if not movable:
                return False
            b = self.rng.choice(movable)
            self.pending[b][1]()
            try:
                self.pending[b] = next(self.wgs[b])
            except StopIteration:
                self.pending[b] = None
                live.remove(b)
                if queued < nwg:                  # its slot goes to the next workgroup
                    live.append(queued)
                    queued += 1
        return len(self.agg) == self.N and queued == nwg


@pytest.mark.parametrize("A,A2", [(2, 2), (4, 3), (3, 5), (1, 2), (8, 1)])
def test_every_schedule_finishes(A, A2):
    for seed in range(40):
        rng = random.Random(seed)
        ntiles = rng.randint(1, 900)
        nwg = rng.choice([1, 2, 3, 8, 13, 40, 96])
        assert Model(ntiles, A, A2, nwg, True, seed).run(), (A, A2, ntiles, nwg, seed)


def test_the_carry_forwarded_from_the_finish_can_deadlock():
    # the earlier schedule: some interleaving leaves every workgroup waiting
    found = False
    for seed in range(200):
        rng = random.Random(1000 + seed)
        ntiles = rng.randint(200, 900)
        if not Model(ntiles, 2, 2, 64, False, seed).run():
            found = True
            break
    assert found


@pytest.mark.parametrize("A,A2", [(2, 2), (4, 3), (256, 256), (1, 1)])
def test_grids_beyond_the_resident_count_finish(A, A2):
    # more workgroups than fit at once: 1x to 16x the resident count, which itself ranges from
    # a single workgroup to many; the waiting ones claim tiles only when they start
    for seed in range(40):
        rng = random.Random(5000 + seed)
        ntiles = rng.randint(1, 700)
        resident = rng.choice([1, 2, 3, 8, 9, 24, 64])
        nwg = resident * rng.choice([1, 2, 4, 16])
        assert Model(ntiles, A, A2, nwg, True, seed, resident).run(), (A, A2, ntiles, nwg,
                                                                       resident, seed)


def test_more_counters_than_resident_workgroups_can_stall():
    # why the host caps the counters at the resident count: 8 counters, 3 resident workgroups
    m = Model(239, 2, 2, 48, True, 0, resident=3)
    m.nc = 8
    m.wgs = [m.program(b) for b in range(48)]
    m.pending = [next(w) for w in m.wgs]
    assert not m.run()


def run_shared(grids, per_xcd, rng):
    """Two or more grids on one chip of 8 XCDs with per_xcd slots each: workgroup b of a grid
    goes to XCD b mod 8, each XCD starts its share of each grid in index order and fills a free
    slot with the next queued workgroup of a grid picked at random.  True if every grid
    finishes; False at the first state where nothing can move."""
    queued = [[[b for b in range(len(g.wgs)) if b % 8 == x] for x in range(8)] for g in grids]
    free = [per_xcd] * 8
    live = []                                      # (grid, workgroup, xcd)

    def fill():
        for x in range(8):
            while free[x] > 0:
                cand = [gi for gi in range(len(grids)) if queued[gi][x]]
                if not cand:
                    break
                gi = rng.choice(cand)
                live.append((gi, queued[gi][x].pop(0), x))
                free[x] -= 1

    fill()
    while live:
        movable = [e for e in live if grids[e[0]].ready(grids[e[0]].pending[e[1]][0])]
        if not movable:
            return False
        gi, b, x = rng.choice(movable)
        g = grids[gi]
        g.pending[b][1]()
        try:
            g.pending[b] = next(g.wgs[b])
        except StopIteration:
            g.pending[b] = None
            live.remove((gi, b, x))
            free[x] += 1
            fill()
    return all(len(g.agg) == g.N for g in grids)


def shared_grids(by_rank, seed, per_xcd_choices=(1, 2, 3)):
    rng = random.Random(seed)
    per_xcd = rng.choice(per_xcd_choices)
    grids = [Model(rng.randint(60, 400), rng.choice([2, 3]), 2, 8 * per_xcd, True, seed + 17 * k,
                   by_rank=by_rank) for k in range(2)]   # each grid alone fills the chip
    return grids, per_xcd, rng


def test_two_scans_with_index_counters_can_deadlock():
    # the earlier counter choice (b mod nc): some interleaving of two full-chip scans stalls
    assert any(not run_shared(*shared_grids(False, seed)) for seed in range(200))


def test_two_scans_with_rank_counters_always_finish():
    # 16 or 24 slots per XCD: at least nc = 8 per scan
    for seed in range(200):
        grids, per_xcd, rng = shared_grids(True, seed, (16, 24))
        assert run_shared(grids, per_xcd, rng), seed


def test_rank_counters_need_nc_slots_per_scan():
    # one slot per XCD for two scans of 8 counters: both can stop short
    assert any(not run_shared(*shared_grids(True, seed, (1,))) for seed in range(200))
