"""The streamed walk's schedule (moe_walk_plan, host only, no GPU) against the rules the Strata
prompt-path page "Prompt path: an MMQ group's experts gathered in one launch, after one wait,
released by one event" sets in "What changes":

  - one gather launch per group (a skipped ring entry inside an open group launches what the
    group holds so far);
  - one wait per batch, on the batch's last copy (the copy stream is in order);
  - one event per batch, releasing every ring slot the batch read; a copy that refills a slot
    waits on used[used_of[slot]], and an event recorded again later only delays that copy;
  - a slot is never refilled before the batch that reads it has been launched;
and, with the CPU share ("#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto ...", "What it does":
the host takes some streamed experts and the GPU the rest), an expert the host computes is
neither copied nor gathered, and no batch spans its position.

The checker below replays the op list the library returns with its own model of the two streams
and the events; it shares nothing with the planner but the op encoding of include/moe_prefill.h.
"""
import numpy as np
import pytest

from quantized_expert_grouped_amd import abi

OP_COPY, OP_GATHER, OP_MMQ = abi.OP_COPY, abi.OP_GATHER, abi.OP_MMQ
EV = abi.WALK_EVENTS


class Sim:
    """Slot contents and event records that persist across calls of one walk."""

    def __init__(self, n_slots):
        self.n_slots = n_slots
        self.slot_expert = [None] * n_slots     # expert whose bytes the slot holds
        self.slot_reader = [None] * n_slots     # serial of the last batch that read the slot
        self.event_serial = {}                  # event -> serial of the batch that last recorded it
        self.serial = 0


def check_call(sim, ops, counts, ring_start, streamed, G, flags):
    """Replays one call's ops; raises AssertionError naming the first broken rule."""
    E = len(counts)
    ring = [(ring_start + i) % E for i in range(E)]
    routed = [e for e in ring if counts[e] > 0]
    n_active = len(routed)
    pos_of_ring = {}
    for i, e in enumerate(ring):
        if counts[e] > 0:
            pos_of_ring[e] = len(pos_of_ring)
    gathered = [False] * n_active
    copy_of_pos = {}              # position -> slot its copy went to (this call)
    open_slots = set()            # slots copied for positions not yet gathered
    batches = []
    mmq_groups = []
    for k, op in enumerate(ops):
        kind = int(op[0])
        if kind == OP_COPY:
            pos, e, s, wait = (int(v) for v in op[1:5])
            assert 0 <= pos < n_active and routed[pos] == e, f"op {k}: copy of a wrong expert"
            assert streamed[e] != 2, f"op {k}: copy of an expert the host computes"
            assert streamed[e], f"op {k}: copy of a resident expert"
            assert 0 <= s < sim.n_slots, f"op {k}: slot out of range"
            assert s not in open_slots, f"op {k}: slot {s} refilled before its batch was launched"
            reader = sim.slot_reader[s]
            if reader is None:
                assert wait == -1 or wait in sim.event_serial, f"op {k}: wait on a never-recorded event"
            else:
                assert wait >= 0, f"op {k}: slot {s} refilled without waiting for its reader"
                assert sim.event_serial.get(wait, -1) >= reader, \
                    f"op {k}: the awaited event does not cover slot {s}'s last reader"
            assert pos not in copy_of_pos, f"op {k}: position copied twice"
            sim.slot_expert[s] = e
            copy_of_pos[pos] = s
            open_slots.add(s)
        elif kind == OP_GATHER:
            first, n, waits, ev, why = (int(v) for v in op[1:6])
            assert n >= 1 and 0 <= first and first + n <= n_active, f"op {k}: batch out of range"
            assert first // G == (first + n - 1) // G, f"op {k}: batch crosses a group"
            assert 0 <= ev < EV
            has_copy = False
            for p in range(first, first + n):
                assert not gathered[p], f"op {k}: position {p} gathered twice"
                gathered[p] = True
                e = routed[p]
                assert streamed[e] != 2, f"op {k}: gather of an expert the host computes"
                if streamed[e]:
                    s = copy_of_pos.get(p)
                    assert s is not None, f"op {k}: streamed position {p} has no copy"
                    assert sim.slot_expert[s] == e, f"op {k}: slot {s} no longer holds expert {e}"
                    has_copy = True
                else:
                    assert p not in copy_of_pos
            assert waits == int(has_copy), f"op {k}: one wait exactly when the batch copied"
            if flags & abi.WALK_GATHER_ONE:
                assert n == 1, f"op {k}: one-expert mode launched {n}"
            if not flags & abi.WALK_NO_SKIP_FLUSH:
                for p in range(first, first + n - 1):
                    a, b = ring.index(routed[p]), ring.index(routed[p + 1])
                    assert b == a + 1, f"op {k}: batch spans a skipped ring entry"
            for p in range(first, first + n):
                if p in copy_of_pos:
                    s = copy_of_pos[p]
                    sim.slot_reader[s] = sim.serial
                    open_slots.discard(s)
            sim.event_serial[ev] = sim.serial
            sim.serial += 1
            batches.append((first, n, why))
        elif kind == OP_MMQ:
            g, first, n = (int(v) for v in op[1:4])
            assert first == g * G and n == min(G, n_active - first), f"op {k}: wrong MMQ group"
            assert all(gathered[p] or streamed[routed[p]] == 2 for p in range(first, first + n)), \
                f"op {k}: MMQ before its group was gathered"
            assert not mmq_groups or mmq_groups[-1] == g - 1
            mmq_groups.append(g)
        else:
            raise AssertionError(f"op {k}: unknown kind {kind}")
    host = [streamed[e] == 2 for e in routed]
    assert all(g or h for g, h in zip(gathered, host)), "a routed expert was never gathered"
    assert mmq_groups == list(range((n_active + G - 1) // G)), "a group's MMQ is missing"
    assert not open_slots
    return batches


def _case(rng, E, zero_frac):
    counts = rng.integers(1, 50, E).astype(np.int32)
    counts[rng.random(E) < zero_frac] = 0
    if counts.sum() == 0:
        counts[rng.integers(E)] = 3
    return counts


def _order(counts, ring_start):
    E = len(counts)
    ring = [(ring_start + i) % E for i in range(E)]
    return [e for e in ring if counts[e] > 0]


def _plan(counts, ring_start, streamed, G, n_slots, flags, state):
    order = _order(counts, ring_start)
    n, ops, state = abi.walk_plan(counts, order, len(order), ring_start, streamed, G, n_slots,
                                  flags, state)
    assert n >= 0, abi.STATUS.get(n, n)
    return ops, state


@pytest.mark.parametrize("E", [1, 7, 64, 512])
@pytest.mark.parametrize("G", [1, 3, 16])
@pytest.mark.parametrize("n_slots", [1, 2, 5, 16, 96])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_schedule_keeps_the_rules(E, G, n_slots, flags):
    rng = np.random.default_rng(E * 1000 + G * 100 + n_slots * 10 + flags)
    sim = Sim(n_slots)
    state = None
    for call in range(3):                       # the slot map and events carry over
        counts = _case(rng, E, zero_frac=[0.0, 0.3, 0.9][call])
        ring_start = int(rng.integers(E))
        streamed = (rng.random(E) < [1.0, 0.5, 0.8][call]).astype(np.uint8)
        ops, state = _plan(counts, ring_start, streamed, G, n_slots, flags, state)
        check_call(sim, ops, counts, ring_start, streamed, G, flags)


def test_one_launch_wait_and_event_per_group_when_nothing_splits_it():
    # every entry routed, a ring deeper than a group: batches are exactly the groups
    E, G = 64, 16
    counts = np.full(E, 5, np.int32)
    ops, _ = _plan(counts, 9, np.ones(E, np.uint8), G, 96, 0, None)
    gathers = [op for op in ops if op[0] == OP_GATHER]
    assert [(int(o[1]), int(o[2]), int(o[3])) for o in gathers] == [(g * G, G, 1) for g in range(4)]
    assert len({int(o[4]) for o in gathers}) == 4          # one event each
    copies = [op for op in ops if op[0] == OP_COPY]
    assert len(copies) == E and all(int(o[4]) == -1 for o in copies)   # a fresh ring: no waits
    # the opt-out: one launch, wait and event per expert
    ops, _ = _plan(counts, 9, np.ones(E, np.uint8), G, 96, abi.WALK_GATHER_ONE, None)
    gathers = [op for op in ops if op[0] == OP_GATHER]
    assert len(gathers) == E and all(int(o[2]) == 1 and int(o[3]) == 1 for o in gathers)


def test_skipped_entry_launches_the_open_group():
    # ring 0..7, entry 3 skipped inside group 0 (positions 0..3 = experts 0, 1, 2, 4)
    counts = np.array([2, 2, 2, 0, 2, 2, 2, 2], np.int32)
    ops, _ = _plan(counts, 0, np.ones(8, np.uint8), 4, 16, 0, None)
    gathers = [(int(o[1]), int(o[2]), int(o[5])) for o in ops if o[0] == OP_GATHER]
    assert gathers == [(0, 3, 1), (3, 1, 0), (4, 3, 0)]
    # without the flush the group stays one batch
    ops, _ = _plan(counts, 0, np.ones(8, np.uint8), 4, 16, abi.WALK_NO_SKIP_FLUSH, None)
    gathers = [(int(o[1]), int(o[2])) for o in ops if o[0] == OP_GATHER]
    assert gathers == [(0, 4), (4, 3)]


def test_ring_smaller_than_a_group_launches_before_reuse():
    counts = np.full(10, 1, np.int32)
    ops, _ = _plan(counts, 0, np.ones(10, np.uint8), 16, 4, 0, None)
    gathers = [(int(o[1]), int(o[2]), int(o[5])) for o in ops if o[0] == OP_GATHER]
    assert gathers == [(0, 4, 2), (4, 4, 2), (8, 2, 0)]
    copies = [int(o[4]) for o in ops if o[0] == OP_COPY]
    assert copies[:4] == [-1] * 4 and copies[4:8] == [0, 0, 0, 0] and copies[8:] == [1, 1]


def test_zipf_routing_with_a_96_slot_ring_never_stalls():
    # many skipped entries (a Zipf-like routing), experts streamed through a 96-slot ring
    rng = np.random.default_rng(5)
    E = 512
    ranks = rng.permutation(E) + 1
    p = ranks ** -1.2
    counts = rng.multinomial(1500, p / p.sum()).astype(np.int32)
    assert (counts == 0).sum() > 100
    sim = Sim(96)
    state = None
    for ring_start in (0, 200, 511):
        ops, state = _plan(counts, ring_start, np.ones(E, np.uint8), 16, 96, 0, state)
        check_call(sim, ops, counts, ring_start, np.ones(E, np.uint8), 16, 0)


def test_checker_catches_planted_mistakes():
    counts = np.full(12, 3, np.int32)
    streamed = np.ones(12, np.uint8)

    def fresh():
        ops, _ = _plan(counts, 0, streamed, 4, 4, 0, None)
        return ops.copy()

    def planted(mutate):
        ops = fresh()
        mutate(ops)
        with pytest.raises(AssertionError):
            check_call(Sim(4), ops, counts, 0, streamed, 4, 0)

    check_call(Sim(4), fresh(), counts, 0, streamed, 4, 0)

    def drop_wait(ops):                  # a refill that does not wait for the slot's reader
        k = [i for i, o in enumerate(ops) if o[0] == OP_COPY and o[4] >= 0][0]
        ops[k, 4] = -1

    def wrong_event(ops):                # waits on an event that never covered the reader
        k = [i for i, o in enumerate(ops) if o[0] == OP_COPY and o[4] >= 0][0]
        ops[k, 4] = (ops[k, 4] + 7) % EV

    def refill_early(ops):               # the second group's first copy before the first launch
        g = [i for i, o in enumerate(ops) if o[0] == OP_GATHER][0]
        c = [i for i, o in enumerate(ops) if o[0] == OP_COPY and i > g][0]
        row = ops[c].copy()
        row[4] = -1
        moved = np.delete(ops, c, axis=0)
        ops[:] = np.insert(moved, g, row, axis=0)

    def no_batch_wait(ops):
        k = [i for i, o in enumerate(ops) if o[0] == OP_GATHER][0]
        ops[k, 3] = 0

    def mmq_too_early(ops):
        m = [i for i, o in enumerate(ops) if o[0] == OP_MMQ][0]
        g = [i for i, o in enumerate(ops) if o[0] == OP_GATHER][0]
        row = ops[m].copy()
        moved = np.delete(ops, m, axis=0)
        ops[:] = np.insert(moved, g, row, axis=0)

    for mutate in (drop_wait, wrong_event, refill_early, no_batch_wait, mmq_too_early):
        planted(mutate)


def test_plan_rejects_inconsistent_inputs():
    counts = np.array([2, 0, 3], np.int32)
    st = lambda: {"used_of": np.full(2, -1, np.int32), "cursor": 0, "next_event": 0}
    ones = np.ones(3, np.uint8)
    assert abi.walk_plan(counts, [2, 0], 2, 0, ones, 4, 2, 0, st())[0] == -1   # not ring order
    assert abi.walk_plan(counts, [0, 2], 1, 0, ones, 4, 2, 0, st())[0] == -1   # wrong n_active
    assert abi.walk_plan(counts, [0, 2], 2, 0, ones, 17, 2, 0, st())[0] == -1  # group > 16
    assert abi.walk_plan(counts, [0, 2], 2, 0, ones, 4, 2, 8, st())[0] == -1   # unknown flag
    bad = st()
    bad["cursor"] = 2
    assert abi.walk_plan(counts, [0, 2], 2, 0, ones, 4, 2, 0, bad)[0] == -1    # cursor >= slots
    assert abi.walk_plan(counts, [0, 2], 2, 0, ones, 4, 2, 0, st(), max_ops=2)[0] == -3
    n, ops, _ = abi.walk_plan(counts, [2, 0], 2, 2, ones, 4, 2, 0, st())       # ring from 2
    assert n == 4 and [int(o[2]) for o in ops if o[0] == OP_COPY] == [2, 0]


@pytest.mark.parametrize("E", [7, 64, 512])
@pytest.mark.parametrize("G", [1, 3, 16])
@pytest.mark.parametrize("n_slots", [1, 5, 96])
def test_schedule_with_host_experts(E, G, n_slots):
    """Some streamed experts computed by the host (state 2), mixed with resident and streamed
    ones, over three calls that carry the ring's state."""
    rng = np.random.default_rng(E * 77 + G * 7 + n_slots)
    sim = Sim(n_slots)
    state = None
    for call in range(3):
        counts = _case(rng, E, zero_frac=[0.0, 0.3, 0.6][call])
        ring_start = int(rng.integers(E))
        streamed = (rng.random(E) < 0.8).astype(np.uint8)
        streamed[(streamed == 1) & (rng.random(E) < [0.5, 0.1, 0.9][call])] = 2
        ops, state = _plan(counts, ring_start, streamed, G, n_slots, 0, state)
        batches = check_call(sim, ops, counts, ring_start, streamed, G, 0)
        ring = [(ring_start + i) % E for i in range(E)]
        routed = [e for e in ring if counts[e] > 0]
        for first, n, _ in batches:              # no batch spans a host expert's position
            for p in range(first, first + n):
                assert streamed[routed[p]] != 2


def test_host_expert_splits_the_batch():
    # ring 0..7 all routed, group 4, expert 2 computed by the host: batches (0,2) and (3,1)
    counts = np.full(8, 2, np.int32)
    streamed = np.ones(8, np.uint8)
    streamed[2] = 2
    ops, _ = _plan(counts, 0, streamed, 4, 16, 0, None)
    gathers = [(int(o[1]), int(o[2]), int(o[5])) for o in ops if o[0] == OP_GATHER]
    assert gathers == [(0, 2, 4), (3, 1, 0), (4, 4, 0)]
    assert [int(o[2]) for o in ops if o[0] == OP_COPY] == [0, 1, 3, 4, 5, 6, 7]
    assert [(int(o[1]), int(o[2]), int(o[3])) for o in ops if o[0] == OP_MMQ] == [(0, 0, 4),
                                                                                   (1, 4, 4)]
    # a whole group computed by the host: no gather for it, its MMQ record still comes
    streamed[4:8] = 2
    ops, _ = _plan(counts, 0, streamed, 4, 16, 0, None)
    assert [(int(o[1]), int(o[2])) for o in ops if o[0] == OP_GATHER] == [(0, 2), (3, 1)]
    assert [int(o[1]) for o in ops if o[0] == OP_MMQ] == [0, 1]


def test_checker_catches_a_gathered_host_expert():
    counts = np.full(8, 2, np.int32)
    streamed = np.ones(8, np.uint8)
    ops, _ = _plan(counts, 0, streamed, 4, 16, 0, None)     # planned as all streamed
    streamed[2] = 2                                          # but checked as host-computed
    with pytest.raises(AssertionError):
        check_call(Sim(16), ops, counts, 0, streamed, 4, 0)


def test_plan_rejects_an_unknown_expert_state():
    counts = np.array([2, 0, 3], np.int32)
    st = {"used_of": np.full(2, -1, np.int32), "cursor": 0, "next_event": 0}
    assert abi.walk_plan(counts, [0, 2], 2, 0, np.array([1, 1, 3], np.uint8), 4, 2, 0, st)[0] == -1
