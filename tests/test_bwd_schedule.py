"""Model of the fused backward's schedule and turn order, on the CPU.

The fused backward (one pass: dK, dV and dQ) runs persistent workgroups
that take (head, key block) items from one queue per XCD, in claim order:
key-block major, so key block 0 of every head of that XCD comes first
(longest first under the causal mask).  An item walks its query blocks from
the last one down (causal: down to the diagonal), and adds its dQ
contribution to query block i only after the previous key block of the same
head has added its own (a turn flag per head, query block and wave slice
counts the contributions made so far).  Each addition is published one step
after it is made.

This model replays that protocol with a discrete-event simulation: W
workers per XCD, random step durations, claims in queue order.  It checks:
  * no deadlock for any worker count, mask, head count or random timing
    (a worker only ever waits on an item claimed before its own);
  * every query block receives its contributions in key-block order, so the
    fp32 sums are formed in one fixed order (bitwise repeatable);
  * the first contribution to every block comes from key block 0, which
    writes instead of adding (no zeroing of dQ needed);
  * heads never cross XCD queues.
A planted mistake (claim order that does not match the turn order) is shown
to deadlock, so the model can fail.
"""
import heapq
import random

import pytest

KB, QB = 256, 32   # keys per item, queries per step


def items_of_xcd(x, nxcd, BH, nkb):
    """Claim order of XCD x's queue: key-block major over the heads h = x mod nxcd."""
    heads = list(range(x, BH, nxcd))
    return [(h, kb) for kb in range(nkb) for h in heads]


def blocks_of_item(kb, nqb, causal):
    lo = kb * (KB // QB) if causal else 0
    return list(range(nqb - 1, lo - 1, -1))


def simulate(BH, S, causal, nxcd, workers, seed, claim_order=None, max_events=2_000_000):
    """Returns (order, deadlocked): order[(h, i)] = list of key blocks in the
    order their contributions to query block i of head h were added."""
    rng = random.Random(seed)
    nkb, nqb = -(-S // KB), -(-S // QB)
    queues = {x: list(items_of_xcd(x, nxcd, BH, nkb)) for x in range(nxcd)}
    if claim_order is not None:
        queues = {x: claim_order(q) for x, q in queues.items()}
    flags = {}            # (h, i) -> contributions published
    order = {}
    # worker state: item, list of remaining blocks, pending publish
    events = []           # (time, seq, worker)
    state = {}
    seq = 0
    for x in range(nxcd):
        for wk in range(workers):
            state[(x, wk)] = None
            heapq.heappush(events, (rng.random(), seq, (x, wk)))
            seq += 1
    waiting = {}          # worker -> (h, i, needed)
    n_events = 0
    while events:
        n_events += 1
        if n_events > max_events:
            return order, True
        t, _, wkr = heapq.heappop(events)
        x = wkr[0]
        st = state[wkr]
        if st is None:
            if not queues[x]:
                continue            # queue drained: the worker exits
            h, kb = queues[x].pop(0)
            assert h % nxcd == x, "a head left its XCD"
            st = state[wkr] = {"h": h, "kb": kb, "blocks": blocks_of_item(kb, nqb, causal), "pending": None}
        h, kb = st["h"], st["kb"]
        if st["pending"] is not None:
            # publish last step's contribution (its stores have completed)
            flags[st["pending"]] = flags.get(st["pending"], 0) + 1
            st["pending"] = None
            for other, (oh, oi, need) in list(waiting.items()):
                if flags.get((oh, oi), 0) >= need:
                    del waiting[other]
                    heapq.heappush(events, (t + rng.random() * 0.1, seq, other))
                    seq += 1
        if not st["blocks"]:
            state[wkr] = None       # item done: claim the next one
            heapq.heappush(events, (t + rng.random() * 0.5, seq, wkr))
            seq += 1
            continue
        i = st["blocks"][0]
        if flags.get((h, i), 0) < kb:
            waiting[wkr] = (h, i, kb)   # turn not reached: sleep until published
            continue
        st["blocks"].pop(0)
        if kb == 0:
            assert (h, i) not in order, "block written twice as first contribution"
        order.setdefault((h, i), []).append(kb)
        st["pending"] = (h, i)
        heapq.heappush(events, (t + 0.5 + rng.random(), seq, wkr))
        seq += 1
    return order, bool(waiting)


@pytest.mark.parametrize("BH,S,causal,nxcd,workers", [
    (16, 4096, False, 8, 32), (16, 4096, True, 8, 32), (8, 3000, True, 8, 3), (8, 1000, False, 8, 1),
    (32, 2048, True, 8, 5), (16, 777, True, 8, 32), (16, 2048, False, 4, 2), (24, 1500, True, 8, 7),
])
def test_turn_order_no_deadlock_and_fixed_order(BH, S, causal, nxcd, workers):
    nkb, nqb = -(-S // KB), -(-S // QB)
    for seed in range(3):
        order, dead = simulate(BH, S, causal, nxcd, workers, seed)
        assert not dead, "deadlock"
        for h in range(BH):
            for i in range(nqb):
                kmax = min(nkb - 1, (i * QB) // KB) if causal else nkb - 1
                assert order[(h, i)] == list(range(kmax + 1)), (h, i, order[(h, i)][:8])


def test_planted_mismatch_deadlocks():
    """Claiming key blocks in the reverse order while the turns stay in key
    block order makes early claimers wait on items nobody can claim: the
    model must report it."""
    order, dead = simulate(8, 4096, False, 8, 2, 0, claim_order=lambda q: q[::-1], max_events=200_000)
    assert dead
