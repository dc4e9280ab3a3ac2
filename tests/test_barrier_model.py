"""A CPU model of the two barrier layouts, explored over every interleaving.

R waiters run `steps` barrier steps.  In step k a waiter arrives at each of the
R-1 others -- one separate atomic add per peer, in any order and at any speed --
and then waits:
  counting -- one signal per waiter; each peer adds 1 to it, the waiter waits for
              k*(R-1) (the DeepEP pull request "make the rail barrier a counting
              barrier", section "Fix");
  per_peer -- one slot per (waiter, peer); peer p adds 1 to slot p, the waiter
              waits for every slot to reach k.

Two properties are checked at the moment a waiter q passes step k:
  identity -- every peer has made its step-k arrival *at q* (what a barrier that
              carries release needs: each peer's prior writes are ordered before
              an arrival q has seen);
  presence -- every peer has made at least one step-k arrival somewhere (it
              reached the barrier).

The pull request (section "Scoped to the rail team") states that an anonymous
count keeps presence but loses identity, because a peer one step ahead can
stand in for a late arrival; the exploration finds that interleaving for R >= 3
and shows per-peer slots keep both.
"""
import functools

import pytest


def explore(R, steps, layout):
    """Return (identity_violated, presence_violated, deadlock_found) over all
    interleavings."""
    peers = [[p for p in range(R) if p != q] for q in range(R)]

    def can_pass(q, k, added):
        # added[p][q]: arrivals p has made at q so far
        if layout == "counting":
            return sum(added[p][q] for p in peers[q]) >= k * (R - 1)
        return all(added[p][q] >= k for p in peers[q])

    found = {"identity": False, "presence": False, "deadlock": False}

    @functools.lru_cache(maxsize=None)
    def dfs(step, mask, added):
        # step[p]: the step p is in (1-based; steps+1 = done); mask[p]: bit q set
        # once p has arrived at q in its current step
        if all(s > steps for s in step):
            return
        moved = False
        for p in range(R):
            k = step[p]
            if k > steps:
                continue
            full = sum(1 << q for q in peers[p])
            if mask[p] != full:
                for q in peers[p]:
                    if mask[p] >> q & 1:
                        continue
                    na = [list(row) for row in added]
                    na[p][q] += 1
                    nm = list(mask)
                    nm[p] |= 1 << q
                    moved = True
                    dfs(step, tuple(nm), tuple(tuple(row) for row in na))
            elif can_pass(p, k, added):
                for o in peers[p]:
                    if added[o][p] < k:
                        found["identity"] = True
                    if step[o] < k or (step[o] == k and mask[o] == 0):
                        found["presence"] = True
                ns = list(step)
                ns[p] += 1
                nm = list(mask)
                nm[p] = 0
                moved = True
                dfs(tuple(ns), tuple(nm), added)
        if not moved:
            found["deadlock"] = True

    zero = tuple(tuple(0 for _ in range(R)) for _ in range(R))
    dfs(tuple([1] * R), tuple([0] * R), zero)
    return found["identity"], found["presence"], found["deadlock"]


@pytest.mark.parametrize("R,steps", [(3, 2), (3, 3), (4, 2)])
def test_counting_barrier_loses_identity_keeps_presence(R, steps):
    identity, presence, deadlock = explore(R, steps, "counting")
    assert identity, "a peer one step ahead should be able to stand in for a late arrival"
    assert not presence
    assert not deadlock


@pytest.mark.parametrize("R,steps", [(2, 3), (3, 2), (3, 3), (4, 2)])
def test_per_peer_barrier_keeps_identity(R, steps):
    identity, presence, deadlock = explore(R, steps, "per_peer")
    assert not identity and not presence and not deadlock


@pytest.mark.parametrize("steps", [1, 2, 4])
def test_two_waiters_counting_is_per_peer(steps):
    """With one peer the anonymous count names it: no stand-in exists."""
    assert explore(2, steps, "counting") == (False, False, False)


def test_one_step_has_no_stand_in():
    """Nobody can be a step ahead within a single step."""
    for R in (3, 4):
        assert explore(R, 1, "counting") == (False, False, False)


def test_held_back_arrivals():
    """The GPU fault-injection schedule, replayed in the model: waiter 0 holds
    back its step-1 and step-2 arrivals at waiter 1 until it has passed step 2.
    Counting with R >= 3 completes with waiter 1 passing step 1 before waiter 0
    arrived there; per-peer slots (and counting with R = 2) cannot progress."""
    def run(R, layout, steps=3):
        added = [[0] * R for _ in range(R)]
        step = [1] * R
        arrived = [0] * R  # the last step each waiter arrived in
        held = 0
        early = False
        progress = True
        while progress and min(step) <= steps:
            progress = False
            for p in range(R):
                k = step[p]
                if k > steps:
                    continue
                if arrived[p] < k:  # arrive once, at the start of the step
                    arrived[p] = k
                    for q in range(R):
                        if q == p:
                            continue
                        if p == 0 and q == 1 and k <= 2:
                            held += 1
                        else:
                            added[p][q] += 1
                need_ok = (sum(added[o][p] for o in range(R) if o != p) >= k * (R - 1)
                           if layout == "counting" else
                           all(added[o][p] >= k for o in range(R) if o != p))
                if need_ok:
                    if p == 1 and k == 1 and added[0][1] == 0:
                        early = True
                    step[p] += 1
                    progress = True
                    if p == 0 and k == 2:
                        added[0][1] += held
                        held = 0
        return min(step) > steps, early

    for R in (3, 4, 8):
        assert run(R, "counting") == (True, True)
        assert run(R, "per_peer")[0] is False
    assert run(2, "counting")[0] is False
