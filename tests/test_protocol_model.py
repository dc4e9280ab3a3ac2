"""A CPU model of the hop hand-off protocol, explored over every interleaving.

Workgroup (r, w) runs hops 1..G: wait (from hop 2 on), work, arrive (up to hop
G-1).  Its hop-g work reads what workgroup (r-1, w) wrote at hop g-1, so the
safety property is: when (r, w) starts hop g, (r-1, w) has finished hop g-1.

Signal layouts:
  lane     -- one signal per (lane w, rank r); only (r-1, w) adds to it in P2P;
              in barrier mode the one workgroup of every other rank in lane w
              adds to it.  This is what the GPU library does.
  team     -- one signal per rank shared by the W workgroups of a team; a
              consumer expects W arrivals per hop (P2P) or (R-1)*W (barrier).

The DeepEP pull request "make the rail barrier a counting barrier" (section
"Scoped to the rail team") notes that an anonymous count can be met by a peer
one round ahead standing in for a late one.  The model finds exactly that
interleaving for the shared team signal and proves the lane layout safe.
"""
import functools

import pytest


def explore(R, W, G, layout, mode):
    """Return True if some interleaving violates the safety property."""
    wgs = [(r, w) for r in range(R) for w in range(W)]
    n = len(wgs)

    def sig_index(r, w):
        return r * W + w if layout == "lane" else r

    nsig = R * W if layout == "lane" else R

    def expected_per_hop():
        if mode == "p2p":
            return 1 if layout == "lane" else W
        return (R - 1) if layout == "lane" else (R - 1) * W

    E = expected_per_hop()

    def targets(r, w):
        if mode == "p2p":
            return [sig_index((r + 1) % R, w)]
        return [sig_index(q, w) for q in range(R) if q != r]

    # per workgroup program counter: step k in 0..3G-1 encodes (hop, phase)
    # phase 0 wait, 1 work, 2 arrive; "done[hop]" tracked as completed work hops
    @functools.lru_cache(maxsize=None)
    def dfs(pcs, sigs, done):
        for i in range(n):
            pc = pcs[i]
            if pc >= 3 * G:
                continue
            hop, phase = pc // 3 + 1, pc % 3
            r, w = wgs[i]
            npcs = list(pcs)
            nsigs = list(sigs)
            ndone = list(done)
            if phase == 0:
                if hop > 1 and sigs[sig_index(r, w)] < (hop - 1) * E:
                    continue  # blocked
                npcs[i] = pc + 1
            elif phase == 1:
                if hop > 1:
                    pred = wgs.index(((r - 1) % R, w))
                    if done[pred] < hop - 1:
                        return True  # starts hop g before its producer finished g-1
                ndone[i] = hop
                npcs[i] = pc + 1
            else:
                if hop < G:
                    for t in targets(r, w):
                        nsigs[t] += 1
                npcs[i] = pc + 1
            if dfs(tuple(npcs), tuple(nsigs), tuple(ndone)):
                return True
        return False

    return dfs(tuple([0] * n), tuple([0] * nsig), tuple([0] * n))


@pytest.mark.parametrize("R,W,G", [(2, 2, 3), (3, 2, 3), (2, 3, 3)])
def test_shared_team_signal_is_unsafe_p2p(R, W, G):
    assert explore(R, W, G, "team", "p2p")


@pytest.mark.parametrize("R,W,G", [(2, 2, 4), (3, 2, 3), (2, 3, 3), (4, 1, 4)])
def test_lane_signals_are_safe_p2p(R, W, G):
    assert not explore(R, W, G, "lane", "p2p")


@pytest.mark.parametrize("R,W,G", [(2, 2, 3), (3, 2, 3)])
def test_shared_team_signal_is_unsafe_barrier(R, W, G):
    assert explore(R, W, G, "team", "barrier")


@pytest.mark.parametrize("R,W,G", [(2, 2, 4), (3, 2, 3), (3, 1, 4), (4, 1, 3)])
def test_lane_signals_are_safe_barrier(R, W, G):
    assert not explore(R, W, G, "lane", "barrier")


def test_one_team_member_is_the_lane_layout():
    # with W = 1 both layouts coincide and both are safe
    assert not explore(3, 1, 4, "team", "p2p")
    assert not explore(3, 1, 4, "team", "barrier")
