"""CPU model check of the cross-workgroup hand-off used by the decode GEMM's split K and the
attention core's cut key ranges.

Protocol (per cut row group / query block, W workgroups):
  1. every workgroup stores its partial (device-scope atomic stores, which gfx950 issues as
     sc1 stores: written through to the agent's coherence point);
  2. it waits until its stores are acknowledged (s_waitcnt vmcnt(0)) and meets its other
     waves at the barrier;
  3. one thread increments the arrival counter (a device-scope atomic add, coherent) and
     learns the previous value;
  4. the workgroup that saw W - 1 is the last: it reads every partial (sc1 loads, issued
     after its add returned), sums them in workgroup order, and resets the counter to 0.

The model makes each store visible only at a separate "ack" event that the scheduler places
anywhere after the store; a load returns the value visible when it runs. Every interleaving
of every workgroup's events is explored for W = 2 and 3: with the wait of step 2 the last
arriver always sums every partial, exactly one workgroup is last, and the counter ends at 0.
Without the wait (the add may run before the stores are acknowledged) some interleaving
reads a missing partial, which shows the wait is the ordering the protocol rests on."""
import itertools


def _explore(W, wait_for_acks):
    """All interleavings; yields the outcome of each: (sum read by the last arriver or None,
    number of last arrivers, final counter)."""
    partial = [10 ** w for w in range(W)]  # distinct digits: a missing one changes the sum
    expect = sum(partial)
    outcomes = []

    def step(state):
        pc, acked, visible, counter, last, reads, trace = state
        moves = []
        for w in range(W):
            # the ack of w's store, any time after the store
            if pc[w] >= 1 and not acked[w]:
                moves.append(("ack", w))
            if pc[w] == 0:
                moves.append(("store", w))
            elif pc[w] == 1 and (acked[w] or not wait_for_acks):
                moves.append(("rmw", w))
            elif pc[w] == 2 and last[w]:
                moves.append(("read", w))
        if not moves:
            return [state]
        done = []
        for kind, w in moves:
            pc2, acked2, vis2, last2, reads2 = list(pc), list(acked), list(visible), list(last), dict(reads)
            counter2 = counter
            if kind == "store":
                pc2[w] = 1
            elif kind == "ack":
                acked2[w] = True
                vis2[w] = partial[w]
            elif kind == "rmw":
                prev = counter2
                counter2 += 1
                last2[w] = prev == W - 1
                pc2[w] = 2
                if last2[w]:
                    counter2 = 0  # the last arriver resets the counter
            elif kind == "read":
                reads2[w] = sum(v for v in vis2)  # loads in workgroup order, visible values
                pc2[w] = 3
            done += step((tuple(pc2), tuple(acked2), tuple(vis2), counter2, tuple(last2), reads2, trace))
        return done

    init = (tuple([0] * W), tuple([False] * W), tuple([0] * W), 0, tuple([False] * W), {}, ())
    for final in step(init):
        pc, acked, visible, counter, last, reads, _ = final
        n_last = sum(last)
        s = next(iter(reads.values())) if reads else None
        outcomes.append((s, n_last, counter, expect))
    return outcomes


def test_handoff_with_store_wait_is_correct_in_every_interleaving():
    for W in (2, 3):
        outs = _explore(W, wait_for_acks=True)
        assert len(outs) > 10
        for s, n_last, counter, expect in outs:
            assert n_last == 1
            assert s == expect
            assert counter == 0


def test_handoff_without_store_wait_can_miss_a_partial():
    for W in (2, 3):
        outs = _explore(W, wait_for_acks=False)
        assert any(s != expect for s, _, _, expect in outs)
        # uniqueness of the last arriver does not depend on the wait
        assert all(n_last == 1 for _, n_last, _, _ in outs)


def test_model_explores_all_event_orders_for_two_workgroups():
    """Sanity of the explorer: with two workgroups and the wait, the number of complete
    interleavings equals a direct count over permutations of the six events that respect
    store < ack < rmw per workgroup and the last arriver's read after its own rmw."""
    outs = _explore(2, wait_for_acks=True)
    events = [("s", 0), ("a", 0), ("r", 0), ("s", 1), ("a", 1), ("r", 1)]
    count = 0
    for perm in itertools.permutations(events):
        pos = {e: i for i, e in enumerate(perm)}
        if all(pos[("s", w)] < pos[("a", w)] < pos[("r", w)] for w in (0, 1)):
            count += 1
    assert len(outs) == count  # the read of the last arriver adds one forced event at the end
