"""Pins for the CPU oracle against things other than itself.

* hand-worked cases in tests/golden/hand_cases.json (values derived by hand
  from the pages and the readings);
* library routines for the special cases that reduce to them: numpy lexsort
  for ranking, scipy's softmax for gates, numpy cumsum/searchsorted for the
  round-0 prefix rule, torch's float64 linear/silu for the SwiGLU expert and
  the dense (all-experts / no-capacity) form of Eq. 1;
* invariants that hold for any input (no expert over capacity, kept slots are
  original or permitted re-routes, union never grows, dispatch is a stable
  expert-major permutation).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy.special import softmax

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
with open(GOLDEN) as f:
    CASES = json.load(f)


def _layer_inp(c):
    N = c["N"]
    gamma = math.inf if c["gamma"] == "inf" else float(c["gamma"])
    inp = dict(T=c["T"], N=N, k=c["k"], R=c["R"], group=c["group"],
               gamma=gamma, lam=c["lam"], kprime=c["kprime"], rho=c["rho"],
               logits=np.array(c["logits"], dtype=np.float32),
               is_visual=np.array(c["is_visual"], dtype=np.uint8),
               entropy_w=np.array(c["entropy_w"], dtype=np.float32),
               modality=np.array(c["modality"], dtype=np.int8))
    inp["sim"] = np.array(c.get("sim", np.eye(N)), dtype=np.float32)
    inp["prot"] = np.array(c.get("prot", np.zeros((N, N))), dtype=np.uint8)
    return inp


@pytest.mark.parametrize("case", CASES["layer_cases"], ids=lambda c: c["name"])
def test_hand_layer_case(case):
    rt = O.layer_routing(_layer_inp(case))
    for key, want in case["expect"].items():
        if key == "gate_closed_form":
            e = math.e
            np.testing.assert_allclose(rt["gates"], e / (1 + e), rtol=1e-15)
            continue
        got = rt[key]
        if isinstance(want, float):
            assert got == want, key
        else:
            np.testing.assert_array_equal(np.asarray(got), np.array(want),
                                          err_msg=key)


@pytest.mark.parametrize("case", CASES["capacity_cases"],
                         ids=lambda c: c["name"])
def test_hand_capacity_case(case):
    slot_in = np.array(case["slot_in"], dtype=np.int32)
    # router ranks: the post-SERE slots unless the case moved some
    topk = np.array(case.get("topk", case["slot_in"]), dtype=np.int32)
    out, flags, load, _ = O.capacity_assign(
        topk, slot_in, np.array(case["fallback"], dtype=np.int32),
        case["w_q"], case["cap_q"], case["N"], case["R"], case["group"])
    np.testing.assert_array_equal(out, case["expect"]["slot_out"])
    np.testing.assert_array_equal(flags, case["expect"]["flags"])
    np.testing.assert_array_equal(load, case["expect"]["load_q"])


@pytest.mark.parametrize("case", CASES["formula_cases"],
                         ids=lambda c: c["name"])
def test_formula_case(case):
    ew = np.array([float("nan") if v == "nan" else v
                   for v in case["entropy_w"]], dtype=np.float32)
    vis = np.array(case["is_visual"], dtype=np.uint8)
    wq = O.token_weights_q(vis, ew)
    if "w_q" in case["expect"]:
        assert wq == case["expect"]["w_q"]
    if "cap_q" in case["expect"]:
        r_v, _, _, cap = O.capacities(wq, vis, case["T"], case["N"],
                                      case["k"], case["gamma"], case["lam"],
                                      np.array(case["modality"]))
        assert r_v == case["expect"]["r_v"]
        assert cap == case["expect"]["cap_q"]


def test_capacity_off_is_unlimited():
    r_v, _, _, cap = O.capacities([65536] * 4, np.zeros(4, np.uint8), 4, 2, 1,
                                  math.inf, 1.0, np.array([1, -1]))
    assert cap is None


def test_all_text_capacity_closed_form():
    # R_v = 0 for an all-text batch, so C_j = base * (1 - lam*m_j/2).
    T, N, k, gamma, lam = 96, 4, 2, 1.25, 1.0
    m = np.array([1, -1, 0, 1])
    _, _, _, cap = O.capacities([65536] * T, np.zeros(T, np.uint8), T, N, k,
                                gamma, lam, m)
    base = gamma * T * k / N          # 60.0 exactly
    want = [int(base * (1 - lam * mj / 2) * 65536) for mj in m]
    assert cap == want


# ----------------------------------------------------------------- ranking
def _tie_logits(rng, T, N):
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0], dtype=np.float32)
    return vals[rng.integers(0, len(vals), size=(T, N))]


@pytest.mark.parametrize("seed", range(6))
def test_route_matches_lexsort_and_softmax(seed):
    rng = np.random.default_rng(seed)
    T, N, k, R = 40, 12, 3, 4
    logits = (_tie_logits(rng, T, N) if seed % 2
              else rng.standard_normal((T, N)).astype(np.float32))
    topk, gates, fb = O.route(logits, k, R)
    for t in range(T):
        # lexsort: last key primary -> (-logit) ascending then index ascending
        order = np.lexsort((np.arange(N), -logits[t].astype(np.float64)))
        np.testing.assert_array_equal(topk[t], order[:k])
        np.testing.assert_array_equal(fb[t], order[k:k + R])
        p = softmax(logits[t].astype(np.float64))
        np.testing.assert_allclose(gates[t], p[order[:k]], rtol=1e-13)


def test_negative_zero_ties_lower_index():
    logits = np.array([[0.0, -0.0, -0.0, 0.0]], dtype=np.float32)
    topk, _, fb = O.route(logits, 2, 2)
    assert topk.tolist() == [[0, 1]] and fb.tolist() == [[2, 3]]


# -------------------------------------------------------------------- SERE
def _sere_instance(rng, T, N, k):
    logits = rng.standard_normal((T, N)).astype(np.float32)
    topk, _, _ = O.route(logits, k, 0)
    a = rng.uniform(0, 1, size=(N, N))
    a = np.round(a * 8) / 8                    # force similarity ties
    s = np.triu(a, 1)
    s = (s + s.T).astype(np.float32)
    np.fill_diagonal(s, 1.0)
    prot = (rng.uniform(size=(N, N)) < 0.2).astype(np.uint8)
    return topk, s, prot


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), kprime=st.integers(1, 3),
       rho=st.sampled_from([0.0, 0.3, 0.5, 0.625, 0.99]))
def test_sere_characterisation(seed, kprime, rho):
    rng = np.random.default_rng(seed)
    T, N, k = 9, 10, 4
    topk, S, prot = _sere_instance(rng, T, N, k)
    slot, moved, P = O.sere_reroute(topk, kprime, rho, S, prot)
    P = np.array(P)
    assert set(P.tolist()) == set(topk[:, :kprime].ravel().tolist())
    rho32 = np.float32(rho)
    for t in range(T):
        np.testing.assert_array_equal(slot[t, :kprime], topk[t, :kprime])
        for s in range(kprime, k):
            e = topk[t, s]
            if e in P:
                assert slot[t, s] == e and not moved[t, s]
                continue
            row = np.full(N, -np.inf, dtype=np.float32)
            row[P] = S[e, P]
            pstar = int(np.argmax(row))          # first maximum = lowest index
            ok = row[pstar] > rho32 and prot[e, pstar] == 0
            assert slot[t, s] == (pstar if ok else e)
            assert moved[t, s] == ok
    # the union never grows and always contains every primary
    assert set(P.tolist()) <= set(slot.ravel().tolist()) <= set(topk.ravel().tolist())


def test_sere_identity_cases():
    rng = np.random.default_rng(3)
    T, N, k = 12, 10, 4
    topk, S, prot = _sere_instance(rng, T, N, k)
    zero = np.zeros_like(prot)
    # K' = k: no secondaries
    assert (O.sere_reroute(topk, k, 0.0, S, zero)[0] == topk).all()
    # rho at or above every off-diagonal similarity
    off = S[~np.eye(N, dtype=bool)].max()
    assert (O.sere_reroute(topk, 1, float(off), S, zero)[0] == topk).all()
    # every source protected
    assert (O.sere_reroute(topk, 1, 0.0, S, np.ones_like(prot))[0] == topk).all()
    # rho below every similarity, nothing protected: all secondaries land in P
    slot, _, P = O.sere_reroute(topk, 1, -1.0, S, zero)
    assert set(slot.ravel().tolist()) == set(P)


# --------------------------------------------------------------- capacity
def _cap_instance(rng, T, N, k, R, frac_visual=0.5):
    logits = rng.standard_normal((T, N)).astype(np.float32)
    logits[:, 0] += rng.uniform(0, 2)
    topk, gates, fb = O.route(logits, k, R)
    vis = (rng.uniform(size=T) < frac_visual).astype(np.uint8)
    ew = rng.choice([0.0, 0.25, 0.5, 0.75, 1.0], size=T).astype(np.float32)
    return topk, gates, fb, vis, ew


@pytest.mark.parametrize("seed", range(10))
def test_round0_is_longest_feasible_prefix(seed):
    rng = np.random.default_rng(seed)
    T, N, k = 30, 5, 2
    topk, _, fb, vis, ew = _cap_instance(rng, T, N, k, 0)
    wq = O.token_weights_q(vis, ew)
    _, _, _, cap = O.capacities(wq, vis, T, N, k, 0.6, 1.0,
                                rng.integers(-1, 2, size=N))
    out, flags, load, _ = O.capacity_assign(topk, topk, fb, wq, cap, N, 0, N)
    for j in range(N):
        ts = np.argwhere(topk == j)              # row-major: (t, s) order
        w = np.array([wq[t] for t, _ in ts], dtype=np.int64)
        n_keep = int(np.searchsorted(np.cumsum(w), cap[j], side="right"))
        kept = [(int(t), int(s)) for t, s in ts[:n_keep]]
        dropped = [(int(t), int(s)) for t, s in ts[n_keep:]]
        assert all(out[t, s] == j for t, s in kept)
        assert all(out[t, s] == -1 and flags[t, s] == O.FLAG_DROP
                   for t, s in dropped)
        assert load[j] == w[:n_keep].sum()


def _check_invariants(topk, gates, fb, slot_in, wq, cap, out, flags, load,
                      N, k, R, group):
    T = topk.shape[0]
    active = set(slot_in.ravel().tolist())
    # I1: loads within capacity, and equal to the kept weights
    rec = np.zeros(N, dtype=np.int64)
    for t in range(T):
        for s in range(k):
            if out[t, s] >= 0:
                rec[out[t, s]] += wq[t]
    np.testing.assert_array_equal(rec, load)
    if cap is not None:
        assert all(load[j] <= cap[j] for j in range(N))
    # I2: every kept slot is its post-SERE expert or a permitted fallback
    for t in range(T):
        held = [int(out[t, s]) for s in range(k) if out[t, s] >= 0]
        for s in range(k):
            e = int(out[t, s])
            if e < 0:
                assert flags[t, s] & O.FLAG_DROP
                continue
            if e == slot_in[t, s]:
                assert not flags[t, s] & O.FLAG_MACS
            else:
                assert flags[t, s] & O.FLAG_MACS
                assert e in fb[t, :R].tolist() and e in active
                assert e // group == slot_in[t, s] // group
                assert held.count(e) == list(slot_in[t]).count(e) + 1
    # I4: union never grows
    assert set(out[out >= 0].ravel().tolist()) <= active <= set(topk.ravel().tolist())
    if cap is None:   # I8
        assert (out == slot_in).all() and not (flags & (O.FLAG_DROP | O.FLAG_MACS)).any()


@settings(max_examples=80, deadline=None)
@given(seed=st.integers(0, 100_000), gamma=st.sampled_from([0.3, 0.7, 1.0, 1.5, math.inf]),
       R=st.integers(0, 3), group=st.sampled_from([2, 3, 6]),
       frac=st.sampled_from([0.0, 0.5, 1.0]), sere=st.booleans())
def test_capacity_invariants(seed, gamma, R, group, frac, sere):
    rng = np.random.default_rng(seed)
    T, N, k = 24, 6, 2
    topk, gates, fb, vis, ew = _cap_instance(rng, T, N, k, R, frac)
    slot_in = topk
    if sere:        # capacity after SERE (R3): K'=1, a low threshold
        sim, prot = _sere_instance(rng, T, N, k)[1:3]
        slot_in = O.sere_reroute(topk, 1, 0.3, sim, prot)[0]
    wq = O.token_weights_q(vis, ew)
    m = rng.integers(-1, 2, size=N)
    _, _, _, cap = O.capacities(wq, vis, T, N, k, gamma, 1.0, m)
    out, flags, load, _ = O.capacity_assign(topk, slot_in, fb, wq, cap, N, R,
                                            group)
    _check_invariants(topk, gates, fb, slot_in, wq, cap, out, flags, load,
                      N, k, R, group)
    if cap is not None:
        # every expert with a proposer keeps at least its first one (C >= 1)
        for j in set(slot_in.ravel().tolist()):
            assert load[j] > 0 or all(
                wq[t] == 0 for t, s in np.argwhere(slot_in == j))


def test_floor_keeps_union_at_decode():
    # one token, 8 experts of 128: base < 1 would drop everything without
    # the floor; with it every expert keeps its first proposer.
    rng = np.random.default_rng(0)
    topk, gates, fb, vis, ew = _cap_instance(rng, 1, 128, 8, 8)
    wq = O.token_weights_q(vis, ew)
    _, _, _, cap = O.capacities(wq, vis, 1, 128, 8, 1.25, 1.0,
                                np.zeros(128, np.int8))
    out, *_ = O.capacity_assign(topk, topk, fb, wq, cap, 128, 8, 128)
    assert (out == topk).all()


# --------------------------------------------------------------- dispatch
@pytest.mark.parametrize("seed", range(5))
def test_dispatch_is_stable_expert_major(seed):
    rng = np.random.default_rng(seed)
    T, N, k = 50, 7, 3
    slot = rng.integers(-1, N, size=(T, k)).astype(np.int32)
    off, rtok, rslot, srow = O.dispatch(slot, N)
    tt, ss = np.nonzero(slot >= 0)
    ee = slot[tt, ss]
    order = np.lexsort((ss, tt, ee))
    np.testing.assert_array_equal(rtok, tt[order])
    np.testing.assert_array_equal(rslot, ss[order])
    np.testing.assert_array_equal(off, np.concatenate(
        [[0], np.cumsum(np.bincount(ee, minlength=N))]))
    for i, (t, s) in enumerate(zip(rtok, rslot)):
        assert srow[t, s] == i
    assert (srow[slot < 0] == -1).all()


# ------------------------------------------------------ FFN and combine
def _tiny_layer(rng, T=16, H=8, N=4, k=2, I=6):
    return dict(
        T=T, H=H, N=N, k=k, I=I, dtype="f32", R=0, group=N,
        gamma=math.inf, lam=1.0, kprime=0, rho=0.5,
        logits=rng.standard_normal((T, N)).astype(np.float32),
        is_visual=np.zeros(T, np.uint8), entropy_w=np.ones(T, np.float32),
        modality=np.zeros(N, np.int8),
        sim=np.eye(N, dtype=np.float32), prot=np.zeros((N, N), np.uint8),
        x=rng.standard_normal((T, H)).astype(np.float32),
        w13=(0.3 * rng.standard_normal((N, 2 * I, H))).astype(np.float32),
        w2=(0.3 * rng.standard_normal((N, H, I))).astype(np.float32))


def _torch_expert(x, w13, w2):
    """SwiGLU expert from torch's float64 library ops (gate rows first)."""
    F = torch.nn.functional
    I = w13.shape[0] // 2
    x = torch.from_numpy(x.astype(np.float64))
    w1 = torch.from_numpy(w13[:I].astype(np.float64))
    w3 = torch.from_numpy(w13[I:].astype(np.float64))
    w2 = torch.from_numpy(w2.astype(np.float64))
    return F.linear(F.silu(F.linear(x, w1)) * F.linear(x, w3), w2).numpy()


def test_silu_matches_library():
    a = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(
        O.silu(a), torch.nn.functional.silu(torch.from_numpy(a)).numpy(),
        rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("seed", range(3))
def test_dense_all_experts_reduction(seed):
    # k = N, capacity off, SERE off: Eq. 1 is the softmax-weighted sum of
    # every expert, computed here without any routing or dispatch code.
    rng = np.random.default_rng(seed)
    inp = _tiny_layer(rng, k=4)
    _, y = O.layer_forward(inp)
    p = softmax(inp["logits"].astype(np.float64), axis=1)
    want = sum(p[:, [j]] * _torch_expert(inp["x"], inp["w13"][j], inp["w2"][j])
               for j in range(inp["N"]))
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_dense_topk_reduction(seed):
    rng = np.random.default_rng(10 + seed)
    inp = _tiny_layer(rng, k=2)
    _, y = O.layer_forward(inp)
    lg = inp["logits"].astype(np.float64)
    p = softmax(lg, axis=1)
    mask = np.zeros_like(p)
    for t in range(inp["T"]):
        mask[t, np.lexsort((np.arange(inp["N"]), -lg[t]))[:2]] = 1
    want = sum((p * mask)[:, [j]] *
               _torch_expert(inp["x"], inp["w13"][j], inp["w2"][j])
               for j in range(inp["N"]))
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)


def test_identical_experts_and_drops():
    # all experts equal: y_t = (sum of kept gates) * E(x_t); with a tight
    # capacity some slots are dropped and contribute nothing.
    rng = np.random.default_rng(7)
    inp = _tiny_layer(rng, T=24, k=2)
    inp["w13"][:] = inp["w13"][0]
    inp["w2"][:] = inp["w2"][0]
    inp.update(gamma=0.5, R=0, is_visual=np.ones(24, np.uint8),
               entropy_w=rng.choice([0.5, 1.0], size=24).astype(np.float32))
    rt, y = O.layer_forward(inp)
    assert rt["dropped"] > 0
    kept_g = np.where(rt["slot_expert"] >= 0, rt["gates"], 0.0).sum(axis=1)
    want = kept_g[:, None] * _torch_expert(inp["x"], inp["w13"][0], inp["w2"][0])
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-13)


def test_w2_linearity():
    rng = np.random.default_rng(11)
    inp = _tiny_layer(rng)
    _, y1 = O.layer_forward(inp)
    inp2 = dict(inp, w2=inp["w2"] * np.float32(2.0))
    _, y2 = O.layer_forward(inp2)
    np.testing.assert_allclose(y2, 2 * y1, rtol=1e-14, atol=1e-300)
    inp0 = dict(inp, w2=np.zeros_like(inp["w2"]))
    _, y0 = O.layer_forward(inp0)
    assert not y0.any()


def test_sampled_outputs_equal_full():
    rng = np.random.default_rng(12)
    inp = _tiny_layer(rng)
    rt, y = O.layer_forward(inp)
    toks = [3, 0, 15, 7]
    # BLAS may block a 4-row product differently from a 16-row one
    np.testing.assert_allclose(O.layer_outputs(inp, rt, toks), y[toks],
                               rtol=1e-13, atol=1e-16)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x3E80, 0x7F7F],
                    dtype=np.uint16)
    vals = O.decode(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[4] == 0.25
    assert math.copysign(1.0, vals[3]) == -1.0
    assert vals[5] == float(np.float32(3.3895313892515355e38))


# ---------------------------------------------------------------- entropy
# MACS §3.2 Eq. 4-5 (reading R14): the oracle's entropy weights against
# library routines and closed forms.
def _entropy_inputs(seed, T=40, D=96):
    rng = np.random.default_rng(seed)
    scale = rng.uniform(0.2, 4.0, size=(T, 1))
    x = (rng.standard_normal((T, D)) * scale).astype(np.float32)
    vis = (rng.uniform(size=T) < 0.6).astype(np.uint8)
    return x, vis


@pytest.mark.parametrize("seed", [0, 1])
def test_entropy_matches_scipy(seed):
    from scipy.special import softmax
    from scipy.stats import entropy
    x, vis = _entropy_inputs(seed)
    H = O.token_entropy(x, "f32")
    ref = entropy(softmax(x.astype(np.float64), axis=1), axis=1)
    np.testing.assert_allclose(H, ref, rtol=1e-12, atol=1e-12)


def test_entropy_closed_forms():
    D = 64
    # uniform logits: ln D; one dominant logit: ~0; shift invariance
    x = np.zeros((3, D), dtype=np.float32)
    x[1, 5] = 200.0
    x[2] = np.arange(D, dtype=np.float32) * 0.125   # exact, so is x + 8
    H = O.token_entropy(x, "f32")
    assert abs(H[0] - math.log(D)) < 1e-12
    assert H[1] < 1e-60
    H2 = O.token_entropy(x[2:3] + np.float32(8.0), "f32")
    assert abs(H2[0] - H[2]) < 1e-12


@pytest.mark.parametrize("seed", [0, 1])
def test_entropy_weight_properties(seed):
    x, vis = _entropy_inputs(seed)
    w, H, mu, sigma = O.entropy_weights(x, vis, "f32", delta=2.0, eps=1e-6)
    v = vis != 0
    assert (w[~v] == 1.0).all()                     # text tokens: full weight
    assert ((w[v] > 0) & (w[v] < 1)).all()
    assert abs(mu - H[v].mean()) < 1e-12
    assert abs(sigma - H[v].std()) < 1e-12          # population std
    order = np.argsort(H[v])                         # higher entropy, lower weight
    assert (np.diff(w[v][order]) <= 1e-15).all()
    # sigmoid of a z-score: z-scores are centred, and w(+a) + w(-a) = 1
    ht = (H[v] - mu) / (sigma + 1e-6)
    np.testing.assert_allclose(w[v], 1.0 / (1.0 + np.exp(2.0 * ht)), rtol=1e-14)
    assert abs(ht.mean()) < 1e-9


def test_entropy_weight_degenerate_batches():
    x, vis = _entropy_inputs(3, T=5)
    w, *_ = O.entropy_weights(x, np.zeros(5, np.uint8), "f32")
    assert (w == 1.0).all()                         # no visual token
    one = np.zeros(5, np.uint8); one[2] = 1
    w, *_ = O.entropy_weights(x, one, "f32")
    assert w[2] == 0.5 and (np.delete(w, 2) == 1.0).all()  # sigma = 0: H~ = 0


# ---------------------------------------------------------------- router
# MACS §3.1, the router network G (reading R17: z_t = W_g x_t, W_g stored
# [N, H]).  The scores are pinned by special inputs whose products are known
# without a matrix product: one-hot tokens pick one weight column, an all-ones
# token sums each expert's row, and sums of tokens give sums of scores.
def _router_case(seed, T=12, H=40, N=7):
    rng = np.random.default_rng(seed)
    x = rng.integers(-4, 5, size=(T, H)).astype(np.float32)
    w = rng.integers(-3, 4, size=(N, H)).astype(np.float32)
    return x, w


@pytest.mark.parametrize("seed", [0, 1])
def test_router_onehot_tokens_pick_weight_columns(seed):
    _, w = _router_case(seed)
    N, H = w.shape
    hot = [3, 0, H - 1, 17]
    x = np.zeros((len(hot), H), dtype=np.float32)
    for t, i in enumerate(hot):
        x[t, i] = 2.0 ** (t - 1)
    z = O.router_logits(x, w, "f32")
    assert z.shape == (len(hot), N)
    for t, i in enumerate(hot):
        assert (z[t] == (2.0 ** (t - 1)) * w[:, i].astype(np.float64)).all()


@pytest.mark.parametrize("seed", [0, 1])
def test_router_ones_token_sums_rows_and_is_additive(seed):
    x, w = _router_case(seed)
    ones = np.ones((1, w.shape[1]), dtype=np.float32)
    z1 = O.router_logits(ones, w, "f32")[0]
    assert (z1 == w.astype(np.float64).sum(axis=1)).all()
    # integer inputs: every product and sum is exact in fp64
    a, b = x[:6], x[6:]
    za, zb = O.router_logits(a, w, "f32"), O.router_logits(b, w, "f32")
    assert (O.router_logits(a + b, w, "f32") == za + zb).all()
    assert (O.router_logits(x, 3.0 * w, "f32") == 3.0 * O.router_logits(x, w, "f32")).all()


def test_router_bf16_inputs_and_expert_permutation():
    x, w = _router_case(5)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)   # small integers: exact
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    assert (O.router_logits(xb, wb, "bf16") == O.router_logits(x, w, "f32")).all()
    # permuting the experts' weight rows permutes the scores and the ranking
    rng = np.random.default_rng(9)
    xr = rng.standard_normal((16, 40)).astype(np.float32)
    wr = rng.standard_normal((7, 40)).astype(np.float32)
    perm = rng.permutation(7)
    z, ids, g, fb = O.router_topk(xr, wr, "f32", 3, 2)
    zp, idsp, gp, fbp = O.router_topk(xr, wr[perm], "f32", 3, 2)
    assert (zp == z[:, perm]).all()
    assert (perm[idsp] == ids).all() and (perm[fbp] == fb).all()
    np.testing.assert_allclose(gp, g, rtol=1e-14)  # the sum's order moves
    # the ranking is the lexsort order of the rounded fp32 scores
    order = np.lexsort((np.arange(7)[None, :].repeat(16, 0), -z.astype(np.float64)), axis=1)
    assert (order[:, :3] == ids).all() and (order[:, 3:5] == fb).all()


# ---------------------------------------------------------------- similarity
# SERE §4.2 (reading R18): Frobenius similarity of per-expert matrices.
def test_similarity_matches_scipy_cosine():
    from scipy.spatial.distance import cdist
    rng = np.random.default_rng(4)
    a = rng.standard_normal((9, 5, 7)).astype(np.float32)
    S = O.frobenius_similarity(a, "f32")
    v = a.reshape(9, -1).astype(np.float64)
    ref = 1.0 - cdist(v, v, metric="cosine")
    np.testing.assert_allclose(S, ref, atol=1e-12)
    assert (np.diag(S) == 1.0).all() and (S == S.T).all()


def test_similarity_closed_forms():
    a = np.zeros((5, 2, 3), dtype=np.float32)
    a[0] = [[1, 2, 0], [0, -1, 3]]
    a[1] = 4.0 * a[0]                      # scaled: similarity 1
    a[2] = -a[0]                           # negated: -1
    a[3, 1, 1] = 5.0                       # overlaps a[0] in one entry (-1)
    # a[4] stays zero: 0 with everyone, 1 with itself
    S = O.frobenius_similarity(a, "f32")
    n0 = math.sqrt(1 + 4 + 1 + 9)
    assert abs(S[0, 1] - 1.0) < 1e-15 and abs(S[0, 2] + 1.0) < 1e-15
    assert abs(S[0, 3] - (-5.0) / (n0 * 5.0)) < 1e-15
    assert (S[4, :4] == 0).all() and (S[:4, 4] == 0).all() and S[4, 4] == 1.0
    # bf16 storage of the same small values gives the same matrix
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    assert (O.frobenius_similarity(bits, "bf16") == S).all()


def test_calibration_activations_are_the_expert_ffn():
    rng = np.random.default_rng(6)
    N, H, I, T = 3, 8, 4, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    w13 = (rng.standard_normal((N, 2 * I, H)) * 0.3).astype(np.float32)
    w2 = (rng.standard_normal((N, H, I)) * 0.3).astype(np.float32)
    A = O.calibration_activations(x, w13, w2, "f32")
    assert A.shape == (N, T, H)
    # torch's float64 SwiGLU of expert 1 as an independent evaluation
    xt = torch.from_numpy(x.astype(np.float64))
    g = torch.nn.functional.linear(xt, torch.from_numpy(w13[1, :I].astype(np.float64)))
    u = torch.nn.functional.linear(xt, torch.from_numpy(w13[1, I:].astype(np.float64)))
    y = torch.nn.functional.linear(torch.nn.functional.silu(g) * u,
                                   torch.from_numpy(w2[1].astype(np.float64)))
    np.testing.assert_allclose(A[1], y.numpy(), rtol=1e-13, atol=1e-15)
    # identical experts have similarity 1
    w13[2], w2[2] = w13[0], w2[0]
    S = O.frobenius_similarity(O.calibration_activations(x, w13, w2, "f32"), "f64")
    assert abs(S[0, 2] - 1.0) < 1e-14
