"""Brute-force pin of the oracle's admission and overflow re-route rules.

The rules (MACS page §1 and Fig. 1: overflow is re-routed locally, else
dropped; §3.1 Eq. 3 and §3.3: per-expert capacity; SERE write-up §4.1: the
re-routed secondaries are the experts the layer runs) are written below as
predicates over a complete outcome of every slot, not as a procedure:

  outcome(t, s) = KEEP            kept by its post-SERE expert in round 0
                | (PLACE, r)      moved to its fallback rank k+r in round r
                | DROP            still unplaced after the last round

Every combination of outcomes is enumerated for tiny inputs (T <= 4,
N <= 4, k <= 2, R <= 2, SERE on and off) and tested against the predicates.
Exactly one combination must satisfy them all, and it must equal what
``capacity_assign`` returns.  Nothing here calls or shares code with the
oracle's capacity routine.

Predicates (readings R8 and R9 of the oracle's header):

  P0  KEEP(t,s)  <=>  the inclusive sum of w_q over every slot (t',s') <=
      (t,s) in (token, slot) order whose post-SERE expert equals this
      slot's is <= that expert's capacity.
  Let A = the set of post-SERE experts of all slots.  Before round r a slot
  stands on fallback[t][r'-1] if it was placed in a round r' < r, else on
  its post-SERE expert; it is pending in round r if it is DROP or placed
  in a round >= r.
  P1  In round r a token with pending slots offers only its lowest pending
      slot s*, to c = fallback[t][r-1], and only if c is in A, c and the
      post-SERE expert of (t,s*) lie in the same group of g experts, and no
      slot of the token stands on c before round r.
  P2  The remaining capacity of expert j before round r is its capacity
      minus the weights of the slots that are KEEP on j and of the slots
      placed on j in earlier rounds.
  P3  An offer of round r to c is admitted  <=>  the inclusive sum of w_q
      over that round's offers to c from tokens t' <= t is <= the
      remaining capacity of c before round r.
  P4  A pending slot is (PLACE, r)  <=>  it is its token's s* of round r,
      the offer is valid (P1) and admitted (P3).
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import moe_oracle as O

KEEP, DROP = "keep", "drop"


def _satisfies(outcome, slot_in, fallback, w_q, cap_q, R, group):
    """True iff the outcome {(t,s): KEEP | ('place', r) | DROP} obeys
    P0-P4."""
    T, k = slot_in.shape
    slots = [(t, s) for t in range(T) for s in range(k)]
    post = {(t, s): int(slot_in[t, s]) for t, s in slots}
    active = set(post.values())

    # P0
    for t, s in slots:
        e = post[(t, s)]
        upto = sum(w_q[t2] for t2, s2 in slots
                   if (t2, s2) <= (t, s) and post[(t2, s2)] == e)
        if (outcome[(t, s)] == KEEP) != (upto <= cap_q[e]):
            return False

    def placed_round(ts):
        o = outcome[ts]
        return o[1] if isinstance(o, tuple) else None

    for r in range(1, R + 1):
        def stands_on(ts):
            pr = placed_round(ts)
            if pr is not None and pr < r:
                return int(fallback[ts[0], pr - 1])
            return post[ts]

        def pending(ts):
            pr = placed_round(ts)
            return outcome[ts] == DROP or (pr is not None and pr >= r)

        # P2
        rem = {}
        for j in range(len(cap_q)):
            used = sum(w_q[t] for t, s in slots
                       if (outcome[(t, s)] == KEEP and post[(t, s)] == j)
                       or (placed_round((t, s)) is not None
                           and placed_round((t, s)) < r
                           and int(fallback[t, placed_round((t, s)) - 1]) == j))
            rem[j] = cap_q[j] - used
        # P1
        offers = []                                   # (t, s*, c), token order
        for t in range(T):
            pend = [s for s in range(k) if pending((t, s))]
            if not pend:
                continue
            s_star = pend[0]
            c = int(fallback[t, r - 1])
            held = {stands_on((t, s)) for s in range(k)}
            if (c in active and c // group == post[(t, s_star)] // group
                    and c not in held):
                offers.append((t, s_star, c))
        # P3
        admitted = set()
        for t, s_star, c in offers:
            upto = sum(w_q[t2] for t2, _, c2 in offers if c2 == c and t2 <= t)
            if upto <= rem[c]:
                admitted.add((t, s_star))
        # P4
        for ts in slots:
            if pending(ts) and ((placed_round(ts) == r) != (ts in admitted)):
                return False
    return True


def _enumerate(slot_in, fallback, w_q, cap_q, R, group):
    """Every outcome that satisfies P0-P4.  Each slot ranges over KEEP,
    (PLACE, 1..R) and DROP; P0 alone decides KEEP for a slot from the
    inputs, so it is applied per slot before the product is formed."""
    T, k = slot_in.shape
    slots = [(t, s) for t in range(T) for s in range(k)]
    choices = []
    for t, s in slots:
        e = int(slot_in[t, s])
        upto = sum(w_q[t2] for t2, s2 in slots
                   if (t2, s2) <= (t, s) and int(slot_in[t2, s2]) == e)
        if upto <= cap_q[e]:
            choices.append([KEEP])
        else:
            choices.append([("place", r) for r in range(1, R + 1)] + [DROP])
    found = []
    for combo in itertools.product(*choices):
        outcome = dict(zip(slots, combo))
        if _satisfies(outcome, slot_in, fallback, w_q, cap_q, R, group):
            found.append(outcome)
    return found


def _expected(outcome, topk, slot_in, fallback, w_q, N):
    T, k = slot_in.shape
    out = np.zeros((T, k), np.int32)
    flags = np.zeros((T, k), np.uint8)
    load = np.zeros(N, np.int64)
    for (t, s), o in outcome.items():
        f = O.FLAG_SERE if slot_in[t, s] != topk[t, s] else 0
        if o == DROP:
            out[t, s] = -1
            f |= O.FLAG_DROP
        else:
            out[t, s] = slot_in[t, s] if o == KEEP else fallback[t, o[1] - 1]
            if o != KEEP:
                f |= O.FLAG_MACS
            load[out[t, s]] += w_q[t]
        flags[t, s] = f
    return out, flags, load


def _tiny_instance(rng, T, N, k, R, sere):
    """Router ranks from a random permutation per token; with ``sere`` the
    secondaries outside the primary union P (rank 1) may move onto a
    member of P, as SERE moves them."""
    ranks = np.array([rng.permutation(N) for _ in range(T)], dtype=np.int32)
    topk, fallback = ranks[:, :k].copy(), ranks[:, k:k + R].copy()
    slot_in = topk.copy()
    if sere and k > 1:
        prim = sorted(set(topk[:, 0].tolist()))
        for t in range(T):
            for s in range(1, k):
                if topk[t, s] not in prim and rng.uniform() < 0.7:
                    slot_in[t, s] = prim[rng.integers(len(prim))]
    w_q = [int(v) for v in rng.choice([0, 16384, 32768, 49152, 65536], size=T)]
    cap_q = [int(v) for v in rng.choice(
        [16384, 32768, 65536, 98304, 131072, 196608], size=N)]
    return topk, slot_in, fallback, w_q, cap_q


def _check(topk, slot_in, fallback, w_q, cap_q, N, R, group):
    found = _enumerate(slot_in, fallback, w_q, cap_q, R, group)
    assert len(found) == 1, f"{len(found)} outcomes satisfy the rules"
    want = _expected(found[0], topk, slot_in, fallback, w_q, N)
    got = O.capacity_assign(topk, slot_in, fallback, w_q, cap_q, N, R, group)
    for name, a, b in zip(("slot_out", "flags", "load_q"), got[:3], want):
        np.testing.assert_array_equal(a, b, err_msg=name)


@settings(max_examples=400, deadline=None)
@given(seed=st.integers(0, 2**32 - 1), T=st.integers(1, 4),
       N=st.integers(2, 4), k=st.integers(1, 2), R=st.integers(0, 2),
       group=st.sampled_from([1, 2, 4]), sere=st.booleans())
def test_capacity_assign_is_the_unique_rule_outcome(seed, T, N, k, R, group,
                                                    sere):
    k = min(k, N)
    R = min(R, N - k)
    rng = np.random.default_rng(seed)
    _check(*_tiny_instance(rng, T, N, k, R, sere), N, R, group)


@pytest.mark.parametrize("seed", range(60))
def test_capacity_assign_full_size_tiny_sere(seed):
    # the largest tiny shape with both fallback rounds and SERE moves; odd
    # seeds split the experts into two locality groups, so a slot SERE moved
    # across groups is re-routed within its new expert's group
    rng = np.random.default_rng(1000 + seed)
    N, k, R = 4, 2, 2
    _check(*_tiny_instance(rng, 4, N, k, R, sere=True), N, R,
           2 if seed % 2 else N)


def test_enumerator_sees_the_hand_cases():
    # the predicates reproduce hand cases H5 (held candidate, two rounds)
    # and H8 (a refused offer blocks a lighter later one) on their own
    fb = np.array([[2, 2], [2, 1], [2, 1]], np.int32)
    slot = np.array([[0, 1], [0, 2], [0, 0]], np.int32)
    (o,) = _enumerate(slot, fb, [65536] * 3, [65536, 65536, 131072], 2, 3)
    out, flags, _ = _expected(o, slot, slot, fb, [65536] * 3, 3)
    np.testing.assert_array_equal(out, [[0, 1], [-1, 2], [2, -1]])
    slot = np.array([[0], [0], [0], [1]], np.int32)
    fb = np.array([[1], [1], [1], [0]], np.int32)
    (o,) = _enumerate(slot, fb, [65536, 65536, 16384, 32768], [65536, 65536],
                      1, 2)
    out, _, _ = _expected(o, slot, slot, fb, [65536, 65536, 16384, 32768], 2)
    np.testing.assert_array_equal(out, [[0], [-1], [-1], [1]])
