"""Host model of the decode kernels' cross-split merge protocol (no GPU).

The decode kernels split a KV head's rows over many workgroups ("splits")
and merge their partial results inside the same launch.  A merging
workgroup may only wait without bound for splits it can prove have
started: a launch need not be resident all at once (other kernels, other
streams, a CU mask), and a workgroup spinning on a split that has not been
dispatched could hold the very compute unit that split needs.

This model replays the protocol's atomic steps (group counters, the tile
word's adds, publishing, merging) in random interleavings on a device with
a random number of resident slots: workgroups are dispatched, in random
order, only into free slots, and a workgroup keeps its slot while it waits.
It checks, for every schedule:
  * every head is merged exactly once;
  * nobody waits for a split that has not started;
  * the group and tile words end at zero;
  * the merge of a declined head falls to the split that completed the last
    group.
The constants and field layout restate those of the kernel's tile word:
bits 0..3 count started groups, bits 4..7 count decided heads, bit 8+h marks
head h's decision.
"""

import random

import pytest

GROUP = 16  # splits per group word (the kernels' kSplitGroup)


class Model:
    # decide_after: a designated merger in place makes its decision add after
    # publishing its own partial (the matrix-core kernel) instead of before
    # (the SIMD-lane and 4-bit kernels)
    def __init__(self, n_split, GT, inplace, rng, decide_after=False):
        self.n, self.GT, self.inplace, self.rng = n_split, GT, inplace, rng
        self.decide_after = decide_after
        self.n_groups = (n_split + GROUP - 1) // GROUP
        self.group = [0] * self.n_groups
        self.tile = 0
        self.started = set()
        self.published = set()
        self.merged = {}
        self.decided = set()
        self.final = self.n_groups | (GT << 4) | (((1 << GT) - 1) << 8)

    def group_size(self, g):
        return min(GROUP, self.n - g * GROUP)

    def last_check(self, after):
        if (after & 0xFFFF) == self.final:
            self.tile = 0

    # ---- agents as generators: each yield is one atomic step -------------
    def split(self, s):
        own = [h for h in range(self.GT) if self.inplace and h % self.n == s]
        g = s // GROUP
        t = self.group[g]; self.group[g] += 1          # group add
        self.started.add(s)
        yield "group add"
        ticket = None
        if t == self.group_size(g) - 1:                 # completed its group
            self.group[g] = 0
            yield "group reset"
            ticket = self.tile; self.tile += 1          # tile add
            yield "tile add"
        decision = None
        if own and not self.decide_after:
            decision = yield from self.decide(own)      # after streaming
        self.published.add(s)
        yield "publish"
        if own and self.decide_after:
            decision = yield from self.decide(own)      # after publishing
        heads = []
        if ticket is not None:
            after = ticket + 1
            if (after & 0xF) == self.n_groups:
                heads += [h for h in range(self.GT) if ticket >> (8 + h) & 1]
            self.last_check(after)
        if own:
            if (decision & 0xF) == self.n_groups:
                heads += own
            self.last_check(decision + ((len(own) << 4) | sum(1 << (8 + h) for h in own)))
        for h in heads:
            yield from self.merge(h, who=("split", s))

    def decide(self, own):
        add = (len(own) << 4) | sum(1 << (8 + h) for h in own)
        decision = self.tile; self.tile += add          # decision add
        self.decided.update(own)
        yield "decision add"
        return decision

    def merge_wg(self, h):
        for _ in range(self.rng.randrange(0, 4)):       # bounded reads of the tile word
            if (self.tile & 0xF) == self.n_groups:
                break
            yield "read tile word"
        add = (1 << 4) | (1 << (8 + h))
        old = self.tile; self.tile += add
        self.decided.add(h)
        yield "decision add"
        self.last_check(old + add)
        if (old & 0xF) == self.n_groups:
            yield from self.merge(h, who=("merger", h))

    def merge(self, h, who):
        # waiting is allowed only with proof that every split has started
        assert len(self.started) == self.n, "%s waits for splits that have not started" % (who,)
        while len(self.published) < self.n:
            yield "poll"
        assert h not in self.merged, "head %d merged twice" % h
        self.merged[h] = who
        yield "merge"


def run(n_split, GT, inplace, seed, decide_after=False):
    rng = random.Random(seed)
    m = Model(n_split, GT, inplace, rng, decide_after)
    pending = [m.split(s) for s in range(n_split)]
    if not inplace:
        pending += [m.merge_wg(h) for h in range(GT)]
    rng.shuffle(pending)
    slots = rng.randint(1, len(pending))
    running = []
    steps = 0
    while pending or running:
        if pending and len(running) < slots and (not running or rng.random() < 0.3):
            running.append(pending.pop())
            continue
        a = rng.choice(running)
        try:
            next(a)
        except StopIteration:
            running.remove(a)
        steps += 1
        assert steps < 200000, "no progress: %d running, %d waiting for a slot" % (len(running), len(pending))
    assert sorted(m.merged) == list(range(GT)), m.merged
    assert m.tile == 0 and all(x == 0 for x in m.group), (m.tile, m.group)
    return m


@pytest.mark.parametrize("decide_after", [False, True])
@pytest.mark.parametrize("inplace", [True, False])
@pytest.mark.parametrize("n_split,GT", [(2, 1), (3, 7), (7, 7), (8, 4), (9, 8), (17, 3), (33, 5), (40, 4), (64, 7), (64, 8), (5, 8)])
def test_protocol_random_schedules(n_split, GT, inplace, decide_after):
    for seed in range(150):
        run(n_split, GT, inplace, seed, decide_after)


@pytest.mark.parametrize("decide_after", [False, True])
def test_declined_heads_fall_to_the_last_group_completer(decide_after):
    # with few slots, designated mergers often decide before every split has
    # started; the split that completes the last group then merges the
    # declined heads
    declined = 0
    for seed in range(300):
        m = run(9, 4, seed % 2 == 0, seed, decide_after)
        declined += sum(1 for who in m.merged.values() if who[0] == "split" and m.inplace is False)
        declined += sum(1 for h, who in m.merged.items() if m.inplace and who != ("split", h % m.n))
    assert declined > 0


class WaitAlways(Model):
    """The protocol this replaced: a designated merger always waits (no proof)."""

    def split(self, s):
        own = [h for h in range(self.GT) if self.inplace and h % self.n == s]
        self.started.add(s)
        yield "start"
        self.published.add(s)
        yield "publish"
        for h in own:
            while len(self.published) < self.n:
                yield "poll"
            self.merged[h] = ("split", s)
            yield "merge"

    def merge_wg(self, h):
        while len(self.published) < self.n:
            yield "poll"
        self.merged[h] = ("merger", h)
        yield "merge"


def test_model_catches_waiting_without_proof():
    # with fewer resident slots than workgroups, mergers that always wait can
    # fill every slot and starve the splits they wait for
    stuck = 0
    for seed in range(100):
        rng = random.Random(seed)
        m = WaitAlways(16, 8, seed % 2 == 0, rng)
        pending = [m.split(s) for s in range(16)] + ([] if m.inplace else [m.merge_wg(h) for h in range(8)])
        rng.shuffle(pending)
        slots, running, steps = rng.randint(1, 8), [], 0
        while (pending or running) and steps < 20000:
            if pending and len(running) < slots and (not running or rng.random() < 0.3):
                running.append(pending.pop())
                continue
            a = rng.choice(running)
            try:
                next(a)
            except StopIteration:
                running.remove(a)
            steps += 1
        stuck += steps >= 20000
    assert stuck > 0
