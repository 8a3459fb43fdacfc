"""CPU oracle: one MoE layer forward with MACS capacity routing and SERE re-routing.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The product path
(the HIP library and its binding) never calls it, and it shares no code,
table or helper with that path.

It is deliberately plain and slow: routing, re-routing, capacity admission
and dispatch are pure-Python loops over tokens and slots in the order the
method is described; the expert FFN and the combine are fp64 numpy products
evaluated one expert at a time.

Sources
  [MACS] "MACS: Modality-Aware Capacity Scaling for Efficient Multimodal MoE
         Inference" (Chinese rendering of the arXiv paper):
         §3.1 Eq. 1 (layer output), Eq. 3 (static capacity);
         §3.2 Eq. 5 (text weight 1), Eq. 6 (effective load);
         §3.3 Eq. 7 (effective visual ratio R_v) and the modality indicator m_j;
         §1 / Fig. 1 (two-stage overflow handling: local re-route, else drop).
  [SERE] Multi-image QA inference write-up ("Wen Yi Wen", dynamic visual token
         compression + SERE expert re-routing): §4.1 (batch union of top-K'
         primaries, secondaries move to the most similar primary above a
         threshold, router weights unchanged, prefill keeps top-K),
         §4.2 (per-layer 0/1 protection matrix blocks protected sources only),
         §4.3 kernel notes (similarity and protection share one layout; the
         protection bit is checked once, when a source is about to move).

Readings where the pages are silent, garbled or truncated (each is also used,
independently implemented, by the GPU path):
  R1  gate = softmax over all N router logits, no renormalisation over top-k
      (Eq. 1 uses G(x)_j as is).
  R2  ranking by fp32 logit descending, ties to the lower expert index,
      -0.0 equal to +0.0; fallback candidates are ranks k+1..k+R.
  R3  order: route -> SERE (decode only) -> capacity -> dispatch -> FFN ->
      combine; capacity sees the experts SERE chose.
  R4  SERE: P = union of every token's ranks 1..K'; a secondary e outside P
      goes to p* = argmax_{p in P} S[e][p] (ties to the lowest p) iff
      fp32 S[e][p*] > fp32 rho and Prot[e][p*] == 0; a blocked p* keeps e
      (no second-best); an e already in P never moves.
  R5  a secondary may land on an expert the token already holds; each slot is
      its own dispatch row.
  R6  token weight in fixed point: w_q = round_half_even(w * 2^16), with
      w = 1 for text and clamp(entropy weight, 0, 1) for visual tokens
      (NaN counts as 1).
  R7  capacity (the formula itself is lost where the MACS page is cut off):
      base = ((gamma * T) * k) / N                       (Eq. 3)
      C_j  = base * (1 + (lam * m_j) * (R_v - 1/2)), floored at 1.0
      C_q  = floor(C_j * 2^16); every step one IEEE double operation, left to
      right, no fused multiply-add; gamma = inf turns capacity off.
      R_v  = W_vis / W_all from the integer sums of w_q (1/2 when W_all = 0).
  R8  round 0: each expert walks its proposers in increasing (token, slot)
      order; a proposer is kept iff the inclusive running sum of w_q over the
      expert's proposers so far is <= C_q (a prefix, even past zero weights).
  R9  overflow re-route: A = experts with at least one round-0 proposer.  In
      round r = 1..R every token with an unplaced overflowed slot offers its
      lowest such slot to c = its router rank k+r, if c is in A, in the same
      locality group (floor(c/g) == floor(e/g)) as the slot's expert e, and
      not currently held by any of the token's slots.  Each expert admits
      that round's offers in token order by the same prefix rule against its
      remaining capacity; the remaining capacity shrinks by what it admitted.
      After round R the unplaced slots are dropped (contribute 0, no gate
      renormalisation).  Gates stay those of the original rank.
  R10 dispatch order: expert-major, then (token, slot) ascending.
  R11 expert FFN: E_j(x) = W2_j (silu(W1_j x) * (W3_j x)), no biases,
      W13_j = [W1_j; W3_j] (gate rows first), silu(a) = a / (1 + e^-a).
  R12 combine: y_t = sum over kept slots, in slot order, of gate * E(x_t).
  R14 entropy weights (MACS §3.2 Eq. 4-5; the page calls the normalisation
      image-level but defines mu and sigma over the batch): z = the token's
      layer input x_t (D = H); H(x) = Shannon entropy (natural log) of
      softmax(z); mu and sigma = mean and population standard deviation of
      H over the batch's visual tokens; H~ = (H - mu) / (sigma + eps);
      w = sigmoid(-delta * H~) for visual tokens, 1 for text tokens.  delta
      and eps are not given by the page: parameters (defaults 1 and 1e-6).
  R18 SERE similarity calibration (SERE §4.2: expert activations on a small
      generic calibration set, a per-layer matrix of Frobenius
      similarities, computed once offline): A_j = E_j(X) [T_cal, H] for a
      calibration batch X, every token through every expert; S[i][j] =
      <A_i, A_j>_F / (||A_i||_F ||A_j||_F) (the cosine of the flattened
      matrices), S[j][j] = 1; an expert whose activations are all zero has
      similarity 0 with every other expert.  The calibration set is
      synthetic (x ~ N(0,1)), like every other input here.
  R17 router scores (MACS §3.1: a router network G scores every expert; its
      form is not given): a bias-free linear map z_t = W_g x_t with W_g
      stored [N, H], one row of H weights per expert, in the activation
      type; the scores are fp32 (the route step's input type).  Here z is
      the exact fp64 product, rounded once to fp32 where the route needs it.
"""
from __future__ import annotations

import math

import numpy as np

KEPT, OVERFLOW, PLACED = 0, 1, 2
FLAG_SERE, FLAG_MACS, FLAG_DROP = 1, 2, 4
W_ONE = 1 << 16           # fixed-point weight of one full token (R6)
CAP_UNLIMITED = None
CAP_CLAMP = 1 << 62       # capacities are clamped here so they fit int64


# --------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------
def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of a stored array (fp32, fp64, or bf16 bit
    patterns)."""
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# entropy-weighted token load  [MACS §3.2 Eq. 4-5; R14]
# --------------------------------------------------------------------------
def token_entropy(x: np.ndarray, dtype: str) -> np.ndarray:
    """H(x_t) = -sum_i p_i ln p_i with p = softmax(x_t), per token, in fp64
    from the exact stored values."""
    z = decode(x, dtype)
    H = np.zeros(z.shape[0])
    for t in range(z.shape[0]):
        row = z[t] - z[t].max()
        e = np.exp(row)
        p = e / e.sum()
        nz = p > 0
        H[t] = -float(np.sum(p[nz] * np.log(p[nz])))
    return H


def entropy_weights(x: np.ndarray, is_visual: np.ndarray, dtype: str,
                    delta: float = 1.0, eps: float = 1e-6):
    """Semantic token weights w (Eq. 5) from the entropy z-score over the
    batch's visual tokens (Eq. 4).  Returns (w float64[T], H float64[T],
    mu, sigma)."""
    H = token_entropy(x, dtype)
    vis = np.asarray(is_visual) != 0
    w = np.ones(len(H))
    mu = sigma = 0.0
    if vis.any():
        hv = H[vis]
        mu = float(hv.mean())
        sigma = float(np.sqrt(np.mean((hv - mu) ** 2)))
        ht = (hv - mu) / (sigma + eps)
        w[vis] = 1.0 / (1.0 + np.exp(delta * ht))
    return w, H, mu, sigma


# --------------------------------------------------------------------------
# router: softmax and ranking  [MACS §3.1 Eq. 1; R1, R2]
# --------------------------------------------------------------------------
def route(logits: np.ndarray, k: int, R: int):
    """Top-k experts, their softmax gates and the next R fallback ranks.

    Returns topk_ids int32[T,k] (rank order), gates float64[T,k] and
    fallback_ids int32[T,R].
    """
    T, N = logits.shape
    topk = np.zeros((T, k), dtype=np.int32)
    fallback = np.zeros((T, R), dtype=np.int32)
    gates = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = [float(v) for v in logits[t]]          # exact fp32 values
        # Python compares -0.0 == +0.0, so equal keys fall to the index
        order = sorted(range(N), key=lambda j: (-row[j], j))
        mx = max(row)
        ex = [math.exp(v - mx) for v in row]
        z = sum(ex)
        for s in range(k):
            topk[t, s] = order[s]
            gates[t, s] = ex[order[s]] / z
        for r in range(R):
            fallback[t, r] = order[k + r]
    return topk, gates, fallback


# --------------------------------------------------------------------------
# router scores  [MACS §3.1, the router network G; R17]
# --------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_gate: np.ndarray, dtype: str) -> np.ndarray:
    """z[t, j] = sum_h W_g[j, h] * x[t, h] in fp64 from the exact stored
    values.  x [T,H], w_gate [N,H]; returns float64[T,N]."""
    return decode(x, dtype) @ decode(w_gate, dtype).T


def router_topk(x: np.ndarray, w_gate: np.ndarray, dtype: str, k: int,
                R: int):
    """route() over the router scores rounded once to fp32.  Returns
    (logits float32[T,N], topk_ids, gates, fallback_ids)."""
    z = router_logits(x, w_gate, dtype).astype(np.float32)
    return (z, *route(z, k, R))


# --------------------------------------------------------------------------
# SERE re-routing  [SERE §4.1, §4.2, §4.3; R4, R5]
# --------------------------------------------------------------------------
def sere_reroute(topk: np.ndarray, kprime: int, rho: float,
                 sim: np.ndarray, prot: np.ndarray):
    """Move secondaries outside the batch's primary union onto the most
    similar primary.  Returns (slot_expert int32[T,k], moved bool[T,k],
    primaries sorted list)."""
    T, k = topk.shape
    primaries = sorted({int(topk[t, s]) for t in range(T)
                        for s in range(kprime)})
    rho32 = float(np.float32(rho))
    slot = topk.astype(np.int32).copy()
    moved = np.zeros((T, k), dtype=bool)
    in_p = set(primaries)
    for t in range(T):
        for s in range(kprime, k):
            e = int(topk[t, s])
            if e in in_p:
                continue
            best, best_sim = None, None
            for p in primaries:                      # ascending: ties -> low p
                v = float(sim[e, p])
                if best is None or v > best_sim:
                    best, best_sim = p, v
            if best is not None and best_sim > rho32 and prot[e, best] == 0:
                slot[t, s] = best
                moved[t, s] = True
    return slot, moved, primaries


# --------------------------------------------------------------------------
# MACS weights and capacity  [MACS Eq. 3, Eq. 5, Eq. 6, Eq. 7, §3.3; R6, R7]
# --------------------------------------------------------------------------
def token_weights_q(is_visual: np.ndarray, entropy_w: np.ndarray) -> list:
    """Fixed-point semantic weight per token: text 1.0, visual clamp(w,0,1)."""
    out = []
    for v, w in zip(is_visual, entropy_w):
        if not v:
            out.append(W_ONE)
            continue
        w = float(w)
        if math.isnan(w):
            w = 1.0
        w = min(max(w, 0.0), 1.0)
        out.append(int(round(w * W_ONE)))           # round() is half-even
    return out


def capacities(w_q: list, is_visual: np.ndarray, T: int, N: int, k: int,
               gamma: float, lam: float, modality: np.ndarray):
    """Effective visual ratio and the per-expert fixed-point capacities.

    Returns (R_v, W_all, W_vis, cap_q) with cap_q None when capacity is off.
    """
    w_all = sum(w_q)
    w_vis = sum(w for w, v in zip(w_q, is_visual) if v)
    r_v = (w_vis / w_all) if w_all > 0 else 0.5     # int/int: correctly rounded
    if math.isinf(gamma):
        return r_v, w_all, w_vis, CAP_UNLIMITED
    base = ((gamma * T) * k) / N
    cap_q = []
    for j in range(N):
        scale = lam * float(int(modality[j]))
        c = base * (1.0 + scale * (r_v - 0.5))
        c = max(c, 1.0)
        cq = c * W_ONE
        cap_q.append(CAP_CLAMP if cq >= CAP_CLAMP else int(math.floor(cq)))
    return r_v, w_all, w_vis, cap_q


def capacity_assign(topk: np.ndarray, slot_in: np.ndarray,
                    fallback: np.ndarray, w_q: list, cap_q, N: int, R: int,
                    group: int):
    """Round-0 admission, R fallback rounds, then drop  [MACS §1 / Fig. 1; R8, R9].

    Returns (slot_out int32[T,k] with -1 = dropped, flags uint8[T,k],
    load_q int64[N], info dict).
    """
    T, k = slot_in.shape
    cur = [[int(slot_in[t, s]) for s in range(k)] for t in range(T)]
    state = [[KEPT] * k for _ in range(T)]
    load = [0] * N
    active = [False] * N
    for t in range(T):
        for s in range(k):
            active[cur[t][s]] = True

    if cap_q is CAP_UNLIMITED:
        for t in range(T):
            for s in range(k):
                load[cur[t][s]] += w_q[t]
    else:
        # round 0: prefix rule per expert in (token, slot) order
        run = [0] * N
        for t in range(T):
            for s in range(k):
                e = cur[t][s]
                run[e] += w_q[t]
                if run[e] <= cap_q[e]:
                    load[e] = run[e]
                else:
                    state[t][s] = OVERFLOW
        rem = [cap_q[j] - load[j] for j in range(N)]
        # fallback rounds
        for r in range(1, R + 1):
            offers = []
            for t in range(T):
                s = next((s for s in range(k) if state[t][s] == OVERFLOW),
                         None)
                if s is None:
                    continue
                c = int(fallback[t, r - 1])
                e = cur[t][s]
                if active[c] and c // group == e // group and c not in cur[t]:
                    offers.append((t, s, c))
            run = [0] * N
            got = [0] * N
            for t, s, c in offers:                   # token order
                run[c] += w_q[t]
                if run[c] <= rem[c]:
                    got[c] = run[c]
                    state[t][s] = PLACED
                    cur[t][s] = c
            for j in range(N):
                rem[j] -= got[j]
                load[j] += got[j]

    slot_out = np.zeros((T, k), dtype=np.int32)
    flags = np.zeros((T, k), dtype=np.uint8)
    n_drop = n_macs = 0
    for t in range(T):
        for s in range(k):
            f = FLAG_SERE if int(slot_in[t, s]) != int(topk[t, s]) else 0
            if state[t][s] == OVERFLOW:
                slot_out[t, s] = -1
                f |= FLAG_DROP
                n_drop += 1
            else:
                slot_out[t, s] = cur[t][s]
                if state[t][s] == PLACED:
                    f |= FLAG_MACS
                    n_macs += 1
            flags[t, s] = f
    info = dict(dropped=n_drop, macs_rerouted=n_macs,
                active=[j for j in range(N) if active[j]])
    return slot_out, flags, np.array(load, dtype=np.int64), info


# --------------------------------------------------------------------------
# dispatch  [R10]
# --------------------------------------------------------------------------
def dispatch(slot_out: np.ndarray, N: int):
    """Expert-major permutation of the kept slots.

    Returns expert_offsets int32[N+1], row_token int32[M], row_slot int32[M],
    slot_row int32[T,k] (-1 for dropped slots).
    """
    T, k = slot_out.shape
    rows = []
    for t in range(T):
        for s in range(k):
            e = int(slot_out[t, s])
            if e >= 0:
                rows.append((e, t, s))
    rows.sort()
    offsets = [0] * (N + 1)
    for e, _, _ in rows:
        offsets[e + 1] += 1
    for j in range(N):
        offsets[j + 1] += offsets[j]
    slot_row = np.full((T, k), -1, dtype=np.int32)
    for i, (e, t, s) in enumerate(rows):
        slot_row[t, s] = i
    return (np.array(offsets, dtype=np.int32),
            np.array([t for _, t, _ in rows], dtype=np.int32),
            np.array([s for _, _, s in rows], dtype=np.int32),
            slot_row)


# --------------------------------------------------------------------------
# SERE similarity calibration  [SERE §4.2; R18]
# --------------------------------------------------------------------------
def frobenius_similarity(acts: np.ndarray, dtype: str) -> np.ndarray:
    """S[i][j] = <A_i, A_j>_F / (||A_i||_F ||A_j||_F) for the N matrices
    A_j = acts[j] (any shape; flattened), in fp64 from the stored values.
    S[j][j] = 1; a zero matrix has similarity 0 with every other one."""
    N = acts.shape[0]
    v = decode(acts, dtype).reshape(N, -1)
    g = v @ v.T
    d = np.sqrt(np.diag(g))
    S = np.zeros((N, N))
    for i in range(N):
        for j in range(N):
            if i == j:
                S[i, j] = 1.0
            elif d[i] > 0 and d[j] > 0:
                S[i, j] = g[i, j] / (d[i] * d[j])
    return S


def calibration_activations(x_cal: np.ndarray, w13: np.ndarray, w2: np.ndarray,
                            dtype: str) -> np.ndarray:
    """A_j = E_j(X) for every expert j and every calibration token, fp64,
    shape [N, T_cal, H]."""
    x64 = decode(x_cal, dtype)
    return np.stack([expert_ffn(x64, decode(w13[j], dtype), decode(w2[j], dtype))
                     for j in range(w13.shape[0])])


# --------------------------------------------------------------------------
# expert FFN and combine  [MACS §3.1 Eq. 1; R11, R12]
# --------------------------------------------------------------------------
def silu(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(x64: np.ndarray, w13_j: np.ndarray, w2_j: np.ndarray):
    """E_j for a block of token rows, all in fp64. w13_j [2I,H], w2_j [H,I]."""
    I = w13_j.shape[0] // 2
    g = x64 @ w13_j[:I].T
    u = x64 @ w13_j[I:].T
    return (silu(g) * u) @ w2_j.T


def combine(tokens, slot_out, slot_row, gates, rows_out, H):
    """y_t = sum over kept slots in slot order of gate * E(x_t) (fp64)."""
    y = np.zeros((len(tokens), H), dtype=np.float64)
    for i, t in enumerate(tokens):
        for s in range(slot_out.shape[1]):
            r = int(slot_row[t, s])
            if r >= 0:
                y[i] += gates[t, s] * rows_out[r]
    return y


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------
def layer_routing(inp: dict) -> dict:
    """Routing half of the layer: route, SERE, capacity, dispatch."""
    T, N, k, R = inp["T"], inp["N"], inp["k"], inp["R"]
    topk, gates, fallback = route(inp["logits"], k, R)
    if inp.get("kprime", 0):
        slot_in, _, primaries = sere_reroute(topk, inp["kprime"], inp["rho"],
                                             inp["sim"], inp["prot"])
    else:
        slot_in, primaries = topk.copy(), None
    w_q = token_weights_q(inp["is_visual"], inp["entropy_w"])
    r_v, w_all, w_vis, cap_q = capacities(
        w_q, inp["is_visual"], T, N, k, inp["gamma"], inp["lam"],
        inp["modality"])
    slot_out, flags, load_q, info = capacity_assign(
        topk, slot_in, fallback, w_q, cap_q, N, R, inp["group"])
    offsets, row_token, row_slot, slot_row = dispatch(slot_out, N)
    return dict(
        topk_ids=topk, gates=gates, fallback_ids=fallback,
        slot_sere=slot_in, primaries=primaries, w_q=np.array(w_q),
        r_v=r_v, w_all=w_all, w_vis=w_vis,
        cap_q=(None if cap_q is None else np.array(cap_q, dtype=np.int64)),
        slot_expert=slot_out, flags=flags, load_q=load_q,
        expert_offsets=offsets, row_token=row_token, row_slot=row_slot,
        slot_row=slot_row,
        union_baseline=len(set(topk.ravel().tolist())),
        union_sere=len(set(slot_in.ravel().tolist())),
        union_final=len(set(slot_out[slot_out >= 0].ravel().tolist())),
        **info)


def layer_outputs(inp: dict, rt: dict, tokens=None) -> np.ndarray:
    """fp64 layer output y for ``tokens`` (all tokens when None).

    Expert weights are widened to fp64 one expert at a time, and only the
    experts the requested tokens use are touched.
    """
    dt = inp["dtype"]
    T, H = inp["T"], inp["H"]
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    slot_out, slot_row = rt["slot_expert"], rt["slot_row"]
    k = slot_out.shape[1]
    need = {}
    for t in tokens:
        for s in range(k):
            e = int(slot_out[t, s])
            if e >= 0:
                need.setdefault(e, []).append(int(slot_row[t, s]))
    rows_out = {}
    for e, rws in sorted(need.items()):
        rws = sorted(set(rws))
        toks = [int(rt["row_token"][r]) for r in rws]
        x64 = decode(inp["x"][toks], dt)
        out = expert_ffn(x64, decode(inp["w13"][e], dt), decode(inp["w2"][e], dt))
        for r, o in zip(rws, out):
            rows_out[r] = o
    return combine(tokens, slot_out, slot_row, rt["gates"], rows_out, H)


def layer_forward(inp: dict, tokens=None):
    """Routing plus fp64 outputs; returns (routing dict, y)."""
    rt = layer_routing(inp)
    return rt, layer_outputs(inp, rt, tokens)
