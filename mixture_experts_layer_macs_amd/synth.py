"""Seeded synthetic inputs for the MoE-layer workloads.

This module only draws random inputs of the right shape, distribution and
layout.  It computes no part of the method: no softmax, no ranking, no
capacity, no expert FFN.  Both the CPU oracle's tests and the GPU path take
their inputs from here, and from nowhere else.

Recipe (per workload, see ``configs.py`` for the knobs):

* router logits: fp32 N(0,1); "zipf" adds b_j = -beta*1.1*ln(rank_j) with the
  rank a seeded permutation of 1..N; "straggler" adds +2.0 to four seeded
  experts; ``skew_expert0`` adds a constant to expert 0's column;
* visual mask: "half" = exactly T/2 visual tokens by seeded permutation,
  "frac:f" = round(f*T) of them, "runs70" = 70 % visual tokens in contiguous
  1024-token image runs (the last run shorter) separated by seeded text gaps,
  "none" = all text;
* per-token entropy weights: visual tokens U(0.1,1.0) or Beta(2,5) in fp32,
  text tokens 1.0;
* expert modality indicator m_j: a seeded permutation gives N/4 experts +1,
  N/4 experts -1 and the rest 0 ("quarters"), or all 0 ("zero");
* similarity matrix: fp32, symmetric, off-diagonal U(0,1), diagonal 1;
* protection matrix: u8, all-ones rows for ``n_protected`` seeded experts;
* x ~ N(0,1) and expert weights ~ N(0,0.02), stored as fp32 or as bf16 bit
  patterns (uint16) rounded to nearest-even;
* router weights W_g [N,H] ~ N(0, 1/H) (so x W_g^T has unit variance, like
  the drawn logits), stored the same way.

Every stream has its own ``numpy.random.SeedSequence`` key, so one input does
not shift when another changes size.  Expert weights use one child seed per
expert and are drawn on a thread pool (numpy's generators release the GIL).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import ZIPF_BETA, Workload

# stream ids
_S_LOGITS, _S_RANK, _S_STRAG, _S_VIS, _S_VISW, _S_MOD, _S_SIM, _S_PROT, \
    _S_X, _S_W13, _S_W2, _S_FEAT, _S_GATE = range(1, 14)


def _rng(seed: int, stream: int, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence(entropy=seed, spawn_key=(stream, layer)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even) and return the bit patterns."""
    import torch  # CPU conversion only; torch's float->bfloat16 is RNE
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def visual_mask(wl: Workload, seed: int, layer: int = 0) -> np.ndarray:
    T = wl.T
    rng = _rng(seed, _S_VIS, layer)
    vis = np.zeros(T, dtype=np.uint8)
    if wl.visual == "none":
        return vis
    if wl.visual == "half":
        vis[rng.permutation(T)[: T // 2]] = 1
        return vis
    if wl.visual.startswith("frac:"):
        f = float(wl.visual.split(":", 1)[1])
        vis[rng.permutation(T)[: int(round(f * T))]] = 1
        return vis
    if wl.visual == "runs70":
        n_vis = int(round(0.7 * T))
        runs = [1024] * (n_vis // 1024)
        if n_vis % 1024:
            runs.append(n_vis % 1024)
        rng.shuffle(runs)
        n_gaps = len(runs) + 1
        n_text = T - n_vis
        interior = n_gaps - 2
        # interior gaps at least one text token so image runs stay separate
        gaps = rng.multinomial(n_text - interior, [1.0 / n_gaps] * n_gaps)
        gaps[1:-1] += 1
        pos = 0
        for i, r in enumerate(runs):
            pos += int(gaps[i])
            vis[pos: pos + r] = 1
            pos += r
        assert pos + int(gaps[-1]) == T and int(vis.sum()) == n_vis
        return vis
    raise ValueError(wl.visual)


def entropy_weights(wl: Workload, vis: np.ndarray, seed: int,
                    layer: int = 0) -> np.ndarray:
    rng = _rng(seed, _S_VISW, layer)
    T = wl.T
    if wl.vis_weight == "uniform":
        w = rng.uniform(0.1, 1.0, size=T)
    elif wl.vis_weight == "beta25":
        w = rng.beta(2.0, 5.0, size=T)
    elif wl.vis_weight == "one":
        w = np.ones(T)
    else:
        raise ValueError(wl.vis_weight)
    w = w.astype(np.float32)
    w[vis == 0] = 1.0
    return w


def router_logits(wl: Workload, seed: int, layer: int = 0,
                  zipf_beta: float | None = None) -> np.ndarray:
    T, N = wl.T, wl.N
    beta = ZIPF_BETA if zipf_beta is None else zipf_beta
    z = _rng(seed, _S_LOGITS, layer).standard_normal((T, N))
    bias = np.zeros(N)
    if wl.logits == "zipf":
        rank = _rng(seed, _S_RANK, layer).permutation(N) + 1
        bias = -beta * 1.1 * np.log(rank.astype(np.float64))
    elif wl.logits == "straggler":
        strag = _rng(seed, _S_STRAG, layer).choice(N, size=4, replace=False)
        bias[strag] = 2.0
    elif wl.logits != "normal":
        raise ValueError(wl.logits)
    bias[0] += wl.skew_expert0
    return (z + bias[None, :]).astype(np.float32)


def router_weights(wl: Workload, seed: int, layer: int = 0) -> np.ndarray:
    """W_g [N,H] ~ N(0, 1/H): one row of H weights per expert."""
    w = _rng(seed, _S_GATE, layer).standard_normal((wl.N, wl.H), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(wl.H))
    return w if wl.dtype == "f32" else f32_to_bf16_bits(w)


def expert_modality(wl: Workload, seed: int, layer: int = 0) -> np.ndarray:
    N = wl.N
    m = np.zeros(N, dtype=np.int8)
    if wl.modality == "zero":
        return m
    perm = _rng(seed, _S_MOD, layer).permutation(N)
    q = N // 4
    m[perm[:q]] = 1
    m[perm[q: 2 * q]] = -1
    return m


def similarity(wl: Workload, seed: int, layer: int = 0) -> np.ndarray:
    N = wl.N
    a = _rng(seed, _S_SIM, layer).uniform(0.0, 1.0, size=(N, N))
    s = np.triu(a, 1)
    s = s + s.T
    np.fill_diagonal(s, 1.0)
    return s.astype(np.float32)


def protection(wl: Workload, seed: int, layer: int = 0) -> np.ndarray:
    N = wl.N
    p = np.zeros((N, N), dtype=np.uint8)
    if wl.n_protected:
        rows = _rng(seed, _S_PROT, layer).choice(N, size=wl.n_protected,
                                                  replace=False)
        p[rows, :] = 1
    return p


def visual_features(T: int, H: int, dtype: str, seed: int,
                    layer: int = 0) -> np.ndarray:
    """Token features with spread-out softmax entropies: row t is
    s_t * N(0,1) with a per-row scale s_t ~ U(0.2, 4.0) (sharper rows have
    lower entropy).  Used for the entropy-weight producer."""
    rng = _rng(seed, _S_FEAT, layer)
    s = rng.uniform(0.2, 4.0, size=(T, 1)).astype(np.float32)
    x = rng.standard_normal((T, H), dtype=np.float32) * s
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def activations(wl: Workload, seed: int, layer: int = 0) -> np.ndarray:
    x = _rng(seed, _S_X, layer).standard_normal((wl.T, wl.H), dtype=np.float32)
    return x if wl.dtype == "f32" else f32_to_bf16_bits(x)


def expert_weights(wl: Workload, seed: int, layer: int = 0,
                   experts=None, threads: int | None = None):
    """(w13[N,2I,H], w2[N,H,I]) ~ N(0,0.02); gate rows 0..I-1, up rows I..2I-1.

    ``experts`` restricts generation to a subset (same values as the full
    draw, since each expert has its own child seed); the result then has
    shape [len(experts), ...].
    """
    N, H, I = wl.N, wl.H, wl.I
    idx = list(range(N)) if experts is None else list(experts)
    ss13 = np.random.SeedSequence(entropy=seed, spawn_key=(_S_W13, layer))
    ss2 = np.random.SeedSequence(entropy=seed, spawn_key=(_S_W2, layer))
    kids13 = ss13.spawn(N)
    kids2 = ss2.spawn(N)
    bf = wl.dtype == "bf16"
    out_dt = np.uint16 if bf else np.float32
    w13 = np.empty((len(idx), 2 * I, H), dtype=out_dt)
    w2 = np.empty((len(idx), H, I), dtype=out_dt)

    def one(i):
        j = idx[i]
        a = np.random.default_rng(kids13[j]).standard_normal(
            (2 * I, H), dtype=np.float32)
        a *= np.float32(0.02)
        b = np.random.default_rng(kids2[j]).standard_normal(
            (H, I), dtype=np.float32)
        b *= np.float32(0.02)
        if bf:
            w13[i] = f32_to_bf16_bits(a)
            w2[i] = f32_to_bf16_bits(b)
        else:
            w13[i] = a
            w2[i] = b

    n_thr = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max(1, n_thr)) as ex:
        list(ex.map(one, range(len(idx))))
    return w13, w2


def make_inputs(wl: Workload, seed: int = 0, layer: int = 0,
                weights: bool = True) -> dict:
    """All inputs of one layer call as numpy arrays, plus the scalar knobs."""
    vis = visual_mask(wl, seed, layer)
    d = dict(
        T=wl.T, H=wl.H, N=wl.N, k=wl.k, I=wl.I, dtype=wl.dtype,
        R=wl.R, group=wl.group, gamma=wl.gamma, lam=wl.lam,
        kprime=wl.kprime, rho=wl.rho,
        logits=router_logits(wl, seed, layer),
        is_visual=vis,
        entropy_w=entropy_weights(wl, vis, seed, layer),
        modality=expert_modality(wl, seed, layer),
        sim=similarity(wl, seed, layer),
        prot=protection(wl, seed, layer),
    )
    if weights:
        d["x"] = activations(wl, seed, layer)
        d["w13"], d["w2"] = expert_weights(wl, seed, layer)
    return d


def is_finite_gamma(g: float) -> bool:
    return not math.isinf(g)
