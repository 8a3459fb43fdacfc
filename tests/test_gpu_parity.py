"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer outputs (expert ids, fallback ids, re-routed slots, flags, loads,
capacities, R_v, dispatch maps) must match bit for bit; gates and the layer
output y within the tolerances stated in gpu_util.  Inputs are the seeded
workloads of the pages' shapes, small variants that still span several GEMM
tiles with ragged tails, and adversarial routing cases (ties, +-0, forced
overflow and drops, full protection, K' = k).  Full-size workloads compare
the whole routing and a sample of output tokens that the oracle evaluates
one by one.
"""
import math

import numpy as np
import pytest

from gpu_util import (assert_routing_equal, assert_y_close, load_binding,
                      needs_gpu, run_gpu_layer, say)
from mixture_experts_layer_macs_amd import configs, synth
from oracle import moe_oracle as O

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    return load_binding()


def _mid_bf16(**kw):
    """Mid-size bf16 layer: several row and column tiles, ragged tails."""
    base = configs.MM_PREFILL.with_(name="mid_bf16", T=600, H=512, N=16, k=4,
                                    I=256, gamma=1.0, R=4, group=16)
    return base.with_(**kw)


FULL_Y_CASES = [
    ("tiny_f32", configs.TINY_F32, 0),
    ("tiny_f32_skew", configs.tiny_variants()["tiny_f32_skew"], 0),
    ("tiny_f32_tight", configs.tiny_variants()["tiny_f32_tight"], 1),
    ("tiny_f32_tight_r0", configs.tiny_variants()["tiny_f32_tight_r0"], 2),
    ("mid_bf16_macs", _mid_bf16(), 0),
    ("mid_bf16_tight", _mid_bf16(gamma=0.6, skew_expert0=2.0), 3),
    ("mid_bf16_group4", _mid_bf16(gamma=0.8, group=4), 4),
    ("mid_bf16_sere", _mid_bf16(kprime=2, n_protected=3, logits="zipf",
                                gamma=math.inf), 5),
    ("mid_bf16_small_decode", _mid_bf16(T=7, kprime=1, n_protected=2,
                                        gamma=1.25), 6),
    ("mid_bf16_h768_i384", _mid_bf16(H=768, I=384, T=300), 7),
    # about 1000 prefill down tiles: each persistent workgroup walks three
    # to five, ragged ones included, so the ring crosses tile boundaries
    ("mid_bf16_multi_tile", _mid_bf16(T=3000, N=64, k=8, H=2048, I=256), 16),
    ("qwen3_decode_b128", configs.QWEN3_DECODE, 0),
    ("qwen3_decode_b128_s1", configs.QWEN3_DECODE, 1),
    ("sweep_layer_macs_b64", configs.SWEEP_LAYER.with_(T=64, kprime=2), 0),
    ("sweep_layer_b1", configs.SWEEP_LAYER.with_(T=1, kprime=1), 0),
    # a few dispatch rows: the 16-row weight panel kernels (gate-up up to 64
    # rows, down up to 16), on both sides of the thresholds
    ("sweep_layer_b2", configs.SWEEP_LAYER.with_(T=2, kprime=0), 1),
    ("sweep_layer_b4", configs.SWEEP_LAYER.with_(T=4, kprime=0), 2),
    ("mid_bf16_skinny_t3", _mid_bf16(T=3, kprime=0), 8),
    ("mid_bf16_skinny_t4_h768", _mid_bf16(T=4, H=768, I=384, gamma=0.7), 9),
    ("mid_bf16_t5", _mid_bf16(T=5), 10),
    ("mid_bf16_t9", _mid_bf16(T=9), 12),
    ("mid_bf16_t17", _mid_bf16(T=17), 15),
    # long reductions in the 16-row panel kernels (32 K slices)
    ("mid_bf16_skinny_h4096", _mid_bf16(T=3, H=4096, I=512, k=2), 13),
    ("mid_bf16_skinny_i4096", _mid_bf16(T=2, H=512, I=4096), 14),
    # one expert with more than 16 rows: several 16-row token tiles
    ("mid_bf16_skinny_k1_t30", _mid_bf16(T=30, k=1, R=2, skew_expert0=10.0,
                                                gamma=math.inf), 11),
    # the 48-layer sweep's layer at batches 1 and 128, half the tokens
    # visual, without SERE and with K'=2 (MACS on in all four)
    ("sweep_b1_vis05_off", configs.SWEEP_LAYER.with_(T=1, kprime=0), 0),
    ("sweep_b1_vis05_k2", configs.SWEEP_LAYER.with_(T=1, kprime=2), 0),
    ("sweep_b128_vis05_off", configs.SWEEP_LAYER.with_(T=128, kprime=0), 0),
    ("sweep_b128_vis05_k2", configs.SWEEP_LAYER.with_(T=128, kprime=2), 0),
]


@pytest.mark.parametrize("name,wl,seed", FULL_Y_CASES, ids=[c[0] for c in FULL_Y_CASES])
def test_layer_parity_all_tokens(name, wl, seed):
    say(f"layer parity {name} seed={seed} T={wl.T} H={wl.H} N={wl.N} k={wl.k} I={wl.I}")
    inp = synth.make_inputs(wl, seed)
    rt = O.layer_routing(inp)
    g = run_gpu_layer(inp)
    assert_routing_equal(g, rt, inp)
    y_ref = O.layer_outputs(inp, rt)
    assert_y_close(g["y"], y_ref, wl.dtype)


SAMPLED_CASES = [
    ("mm_prefill_t8192", configs.MM_PREFILL, 0, 48),
    ("mixtral_decode_t64", configs.MIXTRAL_DECODE, 0, 64),
    ("mixtral_prefill_t4096", configs.MIXTRAL_PREFILL, 0, 24),
]


@pytest.mark.parametrize("name,wl,seed,n_tok", SAMPLED_CASES,
                         ids=[c[0] for c in SAMPLED_CASES])
def test_full_size_parity_sampled(name, wl, seed, n_tok):
    say(f"full-size parity {name} T={wl.T} H={wl.H} N={wl.N} I={wl.I}")
    inp = synth.make_inputs(wl, seed)
    rt = O.layer_routing(inp)
    g = run_gpu_layer(inp)
    assert_routing_equal(g, rt, inp)
    rng = np.random.default_rng(1234)
    T = wl.T
    toks = sorted(set(rng.choice(T, size=min(n_tok, T) - 2, replace=False).tolist())
                  | {0, T - 1})
    # make sure a dropped or re-routed token is among the samples when any
    flagged = np.nonzero((rt["flags"] & (O.FLAG_DROP | O.FLAG_MACS)).any(axis=1))[0]
    if len(flagged):
        toks = sorted(set(toks) | {int(flagged[0]), int(flagged[-1])})
    y_ref = O.layer_outputs(inp, rt, toks)
    assert_y_close(g["y"][toks], y_ref, wl.dtype)


ROUTING_CASES = [
    ("mm_prefill_seed1", configs.MM_PREFILL, 1),
    ("mm_prefill_tight", configs.MM_PREFILL.with_(gamma=0.5, R=2), 2),
    ("mm_prefill_r0", configs.MM_PREFILL.with_(R=0), 3),
    ("qwen3_prefill_sere_off", configs.QWEN3_DECODE.with_(T=2048, kprime=0,
                                                          gamma=1.0), 0),
    ("sweep_b256_k1", configs.SWEEP_LAYER.with_(T=256, kprime=1), 4),
    ("sweep_b8_k2_vis09", configs.SWEEP_LAYER.with_(T=8, kprime=2,
                                                    visual="frac:0.9"), 5),
    ("n100_odd", configs.TINY_F32.with_(T=333, N=100, k=3, R=5, group=25,
                                        gamma=0.7), 6),
    ("n1024_wide", configs.TINY_F32.with_(T=40, N=1024, k=16, R=16,
                                          group=1024, gamma=1.0), 7),
    ("k1_many_tokens", configs.TINY_F32.with_(T=9000, N=8, k=1, R=3, gamma=0.9,
                                              skew_expert0=3.0), 8),
    # 133 token blocks: capacity rounds and dispatch past 128 blocks take
    # the last-workgroup (ticket) path
    ("prefill_133_blocks", configs.MM_PREFILL.with_(T=17000, gamma=0.8), 9),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("name,wl,seed", ROUTING_CASES, ids=[c[0] for c in ROUTING_CASES])
def test_routing_parity(name, wl, seed, fused):
    from mixture_experts_layer_macs_amd import binding as B
    if fused and B.moe_routing_workspace_size(wl.T, wl.N, wl.k, wl.R) == 0:
        pytest.skip("shape not covered by the fused routing launch")
    say(f"routing parity {name} T={wl.T} N={wl.N} k={wl.k} R={wl.R} fused={fused}")
    inp = synth.make_inputs(wl, seed, weights=False)
    rt = O.layer_routing(inp)
    g = run_gpu_layer(inp, tokens_out=False, fused=fused)
    assert_routing_equal(g, rt, inp)


SWEEP_POINTS = [(T, frac, kp) for T in (1, 8, 32, 64, 128, 256)
                for frac in (0.1, 0.5, 0.9) for kp in (0, 1, 2)]


@pytest.mark.parametrize("T,frac,kp", SWEEP_POINTS,
                         ids=[f"b{T}_vis{f}_k{kp}" for T, f, kp in SWEEP_POINTS])
def test_sweep_point_routing_every_layer(T, frac, kp):
    """Every point of the 48-layer decode sweep (batch x visual fraction x
    SERE setting, MACS gamma 1.25, R 8), every layer with its own logits,
    similarity and protection matrices, routed as the sweep routes it (the
    fused launch) and compared bit for bit with the oracle: ids, post-SERE
    slots, final slots, flags, loads, capacities and dispatch maps, so the
    union sizes the sweep reports are the oracle's too."""
    wl = configs.SWEEP_LAYER.with_(T=T, visual=f"frac:{frac}", kprime=kp)
    unions = np.zeros(3)
    for layer in range(wl.layers):
        inp = synth.make_inputs(wl, 0, layer=layer, weights=False)
        rt = O.layer_routing(inp)
        g = run_gpu_layer(inp, tokens_out=False)
        assert_routing_equal(g, rt, inp)
        unions += (rt["union_baseline"], rt["union_sere"], rt["union_final"])
    u = unions / wl.layers
    say(f"sweep point b{T} vis{frac} K'={kp}: {wl.layers} layers bit-exact, "
        f"mean unions {u[0]:.2f} / {u[1]:.2f} / {u[2]:.2f}")


def _hand_inputs(c):
    N = c["N"]
    return dict(
        T=c["T"], H=256, N=N, k=c["k"], I=128, dtype="bf16", R=c["R"],
        group=c["group"], gamma=math.inf if c["gamma"] == "inf" else float(c["gamma"]),
        lam=float(c["lam"]), kprime=c["kprime"], rho=float(c["rho"]),
        logits=np.array(c["logits"], dtype=np.float32),
        is_visual=np.array(c["is_visual"], dtype=np.uint8),
        entropy_w=np.array(c["entropy_w"], dtype=np.float32),
        modality=np.array(c["modality"], dtype=np.int8),
        sim=np.array(c.get("sim", np.eye(N)), dtype=np.float32),
        prot=np.array(c.get("prot", np.zeros((N, N))), dtype=np.uint8))


def _hand_cases():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "hand_cases.json")) as f:
        return json.load(f)["layer_cases"]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("case", _hand_cases(), ids=lambda c: c["name"])
def test_hand_cases_on_gpu(case, fused):
    """The hand-worked routing cases (values derived by hand from the pages
    and the readings) reproduced by the HIP path directly."""
    inp = _hand_inputs(case)
    say(f"hand case {case['name']} fused={fused}")
    g = run_gpu_layer(inp, tokens_out=False, fused=fused)
    M = int(g["expert_offsets"][-1])
    got = dict(g, row_token=g["row_token"][:M], row_slot=g["row_slot"][:M],
               slot_expert=g["slot_expert"])
    for key, want in case["expect"].items():
        if key in ("gate_closed_form", "w_q"):
            continue
        if key == "r_v":
            assert g["r_v"] == want, key
        elif key == "cap_q" and case["gamma"] == "inf":
            continue
        elif key.startswith("union_"):
            src = {"union_baseline": g["topk_ids"], "union_sere": g["slot_sere"],
                   "union_final": g["slot_expert"]}[key]
            assert len(set(src[src >= 0].ravel().tolist())) == want, key
        else:
            np.testing.assert_array_equal(np.asarray(got[key]), np.array(want),
                                          err_msg=key)


FUSED_CASES = [
    ("qwen3_decode_b128", configs.QWEN3_DECODE, 0),
    ("sweep_b1_k1", configs.SWEEP_LAYER.with_(T=1, kprime=1), 1),
    ("sweep_b8_k2", configs.SWEEP_LAYER.with_(T=8, kprime=2), 2),
    ("sweep_b256_k2", configs.SWEEP_LAYER.with_(T=256, kprime=2), 3),
    ("sweep_b256_off", configs.SWEEP_LAYER.with_(T=256, kprime=0), 4),
    ("mixtral_decode", configs.MIXTRAL_DECODE, 5),
    ("tiny_tight", configs.tiny_variants()["tiny_f32_tight"], 6),
    ("n100_odd", configs.TINY_F32.with_(T=333, N=100, k=3, R=5, group=25,
                                        gamma=0.7, kprime=1, n_protected=7,
                                        logits="zipf"), 7),
    ("n1024_wide", configs.TINY_F32.with_(T=40, N=1024, k=16, R=16,
                                          group=1024, gamma=1.0, kprime=4,
                                          n_protected=100), 8),
    ("slots_4096", configs.SWEEP_LAYER.with_(T=512, kprime=2, gamma=0.9), 9),
    ("n99_scalar_rows", configs.TINY_F32.with_(T=50, N=99, k=5, R=3, group=99,
                                               gamma=1.0, kprime=2,
                                               n_protected=5, logits="zipf"), 10),
    ("n50_one_wave", configs.TINY_F32.with_(T=77, N=50, k=4, R=6, group=10,
                                            gamma=0.8, kprime=2,
                                            n_protected=4), 11),
]


@pytest.mark.parametrize("name,wl,seed", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_routing_equals_separate_calls(name, wl, seed):
    """The single fused launch reproduces the four separate calls bit for
    bit (gates included: both run the same device code), and both match the
    oracle."""
    from mixture_experts_layer_macs_amd import binding as B
    assert B.moe_routing_workspace_size(wl.T, wl.N, wl.k, wl.R) > 0, name
    say(f"fused vs separate {name} T={wl.T} N={wl.N} k={wl.k} K'={wl.kprime}")
    inp = synth.make_inputs(wl, seed, weights=False)
    a = run_gpu_layer(inp, tokens_out=False, fused=False)
    b = run_gpu_layer(inp, tokens_out=False, fused=True)
    for key in a:
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), key)
    assert_routing_equal(b, O.layer_routing(inp), inp)


def _adversarial_inputs(seed, T=96, N=12, k=4, R=3):
    rng = np.random.default_rng(seed)
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0], dtype=np.float32)
    logits = vals[rng.integers(0, len(vals), size=(T, N))]
    a = np.round(rng.uniform(0, 1, size=(N, N)) * 8) / 8
    s = np.triu(a, 1)
    sim = (s + s.T).astype(np.float32)
    np.fill_diagonal(sim, 1.0)
    ew = rng.choice([np.float32("nan"), -0.5, 0.0, 0.25, 0.5, 1.0, 1.5],
                    size=T).astype(np.float32)
    return dict(T=T, H=256, N=N, k=k, I=128, dtype="bf16", R=R, group=N,
                gamma=0.8, lam=2.0, kprime=1, rho=0.5, logits=logits,
                is_visual=(rng.uniform(size=T) < 0.6).astype(np.uint8),
                entropy_w=ew,
                modality=rng.integers(-1, 2, size=N).astype(np.int8),
                sim=sim, prot=(rng.uniform(size=(N, N)) < 0.3).astype(np.uint8))


ADV = ["ties", "all_protected", "kprime_eq_k", "rho_low", "no_sere", "cap_off"]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("variant", ADV)
def test_adversarial_routing(variant, fused):
    say(f"adversarial routing {variant} fused={fused}")
    inp = _adversarial_inputs(100 + ADV.index(variant))
    if variant == "all_protected":
        inp["prot"][:] = 1
    elif variant == "kprime_eq_k":
        inp["kprime"] = inp["k"]
    elif variant == "rho_low":
        inp["rho"] = -1.0
    elif variant == "no_sere":
        inp["kprime"] = 0
    elif variant == "cap_off":
        inp["gamma"] = math.inf
    rt = O.layer_routing(inp)
    g = run_gpu_layer(inp, tokens_out=False, fused=fused)
    assert_routing_equal(g, rt, inp)


# Batches of at most 8 tokens and 64 slots take the one-workgroup path of
# the fused launch.  These shapes walk its limits and branches: S and Prot
# copied to LDS (N <= 128; N*N a multiple of 16 or not) or read from memory
# (N > 128), SERE off / on / K' = k, capacity off, R = 0, expert groups,
# capacities tight enough to run the fallback rounds, tied logits and
# similarities, NaN and out-of-range entropy weights.
TINY_CASES = [
    # name, T, N, k, R, group, gamma, K', rho, seed
    ("t1_n12_k4", 1, 12, 4, 3, 12, 0.3, 1, 0.5, 500),
    ("t2_n12_k4_tight", 2, 12, 4, 3, 12, 0.3, 1, 0.25, 501),
    ("t3_n50_groups", 3, 50, 4, 6, 10, 0.5, 2, 0.0, 502),
    ("t5_n12_k8", 5, 12, 8, 4, 12, 0.2, 2, 0.25, 503),
    ("t8_n12_64_slots", 8, 12, 8, 4, 12, 0.3, 1, 0.5, 504),
    ("t8_n128_r8", 8, 128, 8, 8, 128, 0.5, 2, 0.25, 505),
    ("t4_n99_odd", 4, 99, 5, 8, 33, 0.4, 2, 0.0, 506),
    ("t6_n200_sere_from_memory", 6, 200, 6, 8, 200, 0.4, 3, 0.0, 507),
    ("t8_n256_groups", 8, 256, 8, 8, 64, 0.3, 2, 0.0, 508),
    ("t7_cap_off", 7, 40, 8, 8, 40, math.inf, 2, 0.0, 509),
    ("t3_r0", 3, 24, 6, 0, 24, 0.3, 1, 0.0, 510),
    ("t8_sere_off", 8, 64, 8, 8, 16, 0.4, 0, 0.5, 511),
    ("t2_kprime_eq_k", 2, 16, 4, 4, 16, 0.3, 4, 0.0, 512),
    ("t1_k1", 1, 8, 1, 7, 8, 1.0, 1, 0.0, 513),
    ("t8_k1_tight", 8, 9, 1, 8, 9, 0.25, 1, 0.0, 514),
    # many fallback placements (15, 16, 11), and under expert groups (13, 11)
    ("t8_n32_placed", 8, 32, 8, 8, 32, 0.7, 1, 0.25, 902),
    ("t8_n32_placed_sere_off", 8, 32, 8, 8, 32, 0.5, 0, 0.25, 902),
    ("t6_n16_placed", 6, 16, 8, 8, 16, 0.9, 1, 0.25, 900),
    ("t8_n32_placed_groups", 8, 32, 8, 8, 16, 0.9, 0, 0.25, 900),
    ("t8_n16_placed_groups", 8, 16, 4, 8, 8, 1.2, 0, 0.25, 903),
]


@pytest.mark.parametrize("case", TINY_CASES, ids=[c[0] for c in TINY_CASES])
def test_tiny_batch_routing(case):
    """Tiny batches: the fused launch equals the separate calls bit for bit
    (gates included) and the oracle."""
    name, T, N, k, R, group, gamma, kprime, rho, seed = case
    say(f"tiny-batch routing {name} T={T} N={N} k={k} R={R} K'={kprime}")
    inp = _adversarial_inputs(seed, T=T, N=N, k=k, R=R)
    inp.update(group=group, gamma=gamma, kprime=kprime, rho=rho)
    rt = O.layer_routing(inp)
    a = run_gpu_layer(inp, tokens_out=False, fused=False)
    b = run_gpu_layer(inp, tokens_out=False, fused=True)
    for key in a:
        np.testing.assert_array_equal(np.asarray(a[key]), np.asarray(b[key]), key)
    assert_routing_equal(b, rt, inp)


def test_fused_workspace_reuse():
    """One fused-routing workspace serves batches of different sizes and
    routing settings back to back (its control words reset themselves)."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import to_device
    say("fused routing workspace reuse")
    cases = [configs.SWEEP_LAYER.with_(T=200, kprime=2, gamma=0.8),
             configs.SWEEP_LAYER.with_(T=17, kprime=1),
             configs.QWEN3_DECODE]
    N, k = 128, 8
    ws = B.new_workspace(B.moe_routing_workspace_size(200, N, k, 8), "cuda")
    for rep in range(2):
        for i, wl in enumerate(cases):
            inp = synth.make_inputs(wl, 10 + i, weights=False)
            d = to_device(inp, "cuda", weights=False)
            lay = B.Layer(wl.T, 256, N, k, 128, wl.R, torch.bfloat16)
            B.moe_routing_fused(d["logits"], d["is_visual"], d["entropy_w"],
                                d["modality"], d["sim"], d["prot"], k, wl.R,
                                wl.kprime, wl.rho, wl.group, wl.gamma, wl.lam,
                                ws, lay.topk_ids, lay.topk_gates,
                                lay.fallback_ids, lay.slot_sere, lay.cap,
                                lay.disp)
            torch.cuda.synchronize()
            rt = O.layer_routing(inp)
            np.testing.assert_array_equal(lay.cap["slot_out"].cpu().numpy(),
                                          rt["slot_expert"], f"{rep}/{i}")
            np.testing.assert_array_equal(lay.disp["slot_row"].cpu().numpy(),
                                          rt["slot_row"], f"{rep}/{i}")


def test_deterministic_and_workspace_reuse():
    """Two runs are bit-identical, and one workspace serves batches of
    different sizes back to back (its control words reset themselves)."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import to_device
    say("determinism + workspace reuse")
    big = synth.make_inputs(configs.MM_PREFILL.with_(H=256, I=128), 0)
    small = synth.make_inputs(configs.SWEEP_LAYER.with_(T=32, H=256, I=128,
                                                        kprime=2), 0)
    T, N, k = big["T"], big["N"], big["k"]
    ws = B.new_workspace(max(B.moe_capacity_workspace_size(T, N, k), 1 << 20), "cuda")
    wd = B.new_workspace(max(B.moe_dispatch_workspace_size(T, N, k), 1 << 20), "cuda")
    results = []
    for inp in (big, small, big, small):
        d = to_device(inp, "cuda", weights=False)
        ids, gates, fb = B.moe_route(d["logits"], inp["k"], inp["R"])
        cap = B.moe_capacity_assign(ids, ids, fb, d["is_visual"], d["entropy_w"],
                                    d["modality"], inp["N"], inp["R"],
                                    inp["group"], inp["gamma"], inp["lam"], ws)
        disp = B.moe_dispatch(cap["slot_out"], inp["N"], wd)
        torch.cuda.synchronize()
        results.append((cap["slot_out"].cpu().numpy(), cap["load_q"].cpu().numpy(),
                        disp["slot_row"].cpu().numpy()))
    for a, b in zip(results[0], results[2]):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(results[1], results[3]):
        np.testing.assert_array_equal(a, b)
    rt = O.layer_routing(dict(small, kprime=0))
    np.testing.assert_array_equal(results[1][0], rt["slot_expert"])


def test_empty_batch_is_noop():
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    lib = B.library()
    assert lib.moe_route(None, 0, 8, 2, 0, None, None, None, None) == 0
    assert lib.moe_combine(None, None, None, 0, 2, 64, 1, None, None) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_graph_replay_matches_eager(fused):
    """The whole layer captured in a HIP graph: every replay, with eager work
    and synchronisations in between, reproduces the eager result bit for
    bit."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import to_device, torch_elem_dtype
    wl = configs.SWEEP_LAYER.with_(T=96, H=512, I=256, kprime=2, gamma=0.8)
    say(f"graph replay vs eager fused={fused}")
    inp = synth.make_inputs(wl, 3)
    d = to_device(inp, "cuda")
    lay = B.Layer(wl.T, wl.H, wl.N, wl.k, wl.I, wl.R, torch_elem_dtype(wl.dtype))
    args = (d["logits"], d["x"], d["w13"], d["w2"], d["is_visual"],
            d["entropy_w"], d["modality"], d["sim"], d["prot"], wl.kprime,
            wl.rho, wl.gamma, wl.lam, wl.group, fused)
    lay.forward(*args)
    torch.cuda.synchronize()
    ref_y = lay.y.clone()
    ref_slot = lay.cap["slot_out"].clone()
    ref_row = lay.disp["slot_row"].clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        lay.forward(*args)
    for i in range(4):
        lay.y.zero_()
        lay.cap["slot_out"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.y, ref_y), f"replay {i}: y"
        assert torch.equal(lay.cap["slot_out"], ref_slot), f"replay {i}: slots"
        assert torch.equal(lay.disp["slot_row"], ref_row), f"replay {i}: rows"
        lay.forward(*args)           # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(lay.y, ref_y)


@pytest.mark.parametrize("T", [1, 2])
def test_graph_replay_packed_small_batch(T):
    """A decode layer of one or two tokens on packed weights (the one-workgroup
    routing, the GEMVs and the combine folded into the down GEMV, whose
    arrival tickets live in the layer's workspace) captured in a HIP graph:
    every replay, with eager work between replays, reproduces the eager y
    bit for bit, and the tickets are zero after each."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import to_device
    wl = configs.SWEEP_LAYER.with_(T=T, kprime=2)
    say(f"graph replay, packed weights, T={T}")
    inp = synth.make_inputs(wl, 5)
    d = to_device(inp, "cuda")
    p13, p2 = B.moe_pack_weights(d["w13"], d["w2"])
    lay = B.Layer(wl.T, wl.H, wl.N, wl.k, wl.I, wl.R, torch.bfloat16)
    args = (d["logits"], d["x"], p13, p2, d["is_visual"], d["entropy_w"],
            d["modality"], d["sim"], d["prot"], wl.kprime, wl.rho, wl.gamma,
            wl.lam, wl.group)
    tickets = lambda: lay.ws_ffn[: (wl.H // 32) * 4].view(torch.int32)
    lay.forward(*args, panels=True)
    torch.cuda.synchronize()
    ref_y = lay.y.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        lay.forward(*args, panels=True)
    for i in range(4):
        lay.y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.y.view(torch.int16), ref_y.view(torch.int16)), f"replay {i}: y"
        assert int(tickets().abs().sum().item()) == 0, f"replay {i}: tickets"
        lay.forward(*args, panels=True)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(lay.y.view(torch.int16), ref_y.view(torch.int16))
    # the eager result against the oracle's layer
    _, y_ref = O.layer_forward(inp)
    assert_y_close(lay.y.float().cpu().numpy().astype(np.float64), y_ref, "bf16")


ENTROPY_CASES = [
    ("bf16_t8192_h2048", 8192, 2048, "bf16", "runs70", 1.0, 0),
    ("bf16_t333_h768_delta3", 333, 768, "bf16", "half", 3.0, 1),
    ("f32_t256_h128", 256, 128, "f32", "half", 1.0, 2),
    ("bf16_t50_h203_odd", 50, 203, "bf16", "half", 0.5, 3),
    ("bf16_one_visual", 9, 256, "bf16", "one", 1.0, 4),
    ("bf16_all_text", 64, 512, "bf16", "none", 1.0, 5),
]


@pytest.mark.parametrize("name,T,H,dtype,vis,delta,seed", ENTROPY_CASES,
                         ids=[c[0] for c in ENTROPY_CASES])
def test_entropy_weights_parity(name, T, H, dtype, vis, delta, seed):
    """Entropy producer (MACS §3.2 Eq. 4-5) against the fp64 oracle: token
    entropies within 1e-5 relative, weights within 2e-5 absolute (fp32
    accumulation over H terms; the z-score divides by sigma, which these
    features keep near 1)."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import elem_tensor
    say(f"entropy weights {name}")
    x = synth.visual_features(T, H, dtype, seed)
    if vis == "one":
        is_vis = np.zeros(T, np.uint8)
        is_vis[T // 2] = 1
    else:
        wl = configs.MM_PREFILL.with_(T=T, H=H, visual=vis)
        is_vis = synth.visual_mask(wl, seed)
    w_ref, H_ref, mu, sigma = O.entropy_weights(x, is_vis, dtype, delta, 1e-6)
    xd = elem_tensor(x, dtype, "cuda")
    vd = torch.from_numpy(is_vis).cuda()
    ws = B.new_workspace(B.moe_entropy_workspace_size(T), "cuda")
    ent = torch.empty(T, dtype=torch.float32, device="cuda")
    for _ in range(2):  # the workspace is reused without clearing
        w = B.moe_entropy_weights(xd, vd, delta, 1e-6, ws, entropy=ent)
        torch.cuda.synchronize()
        np.testing.assert_allclose(ent.cpu().numpy(), H_ref, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=0, atol=2e-5)
    say(f"mu={mu:.4f} sigma={sigma:.4f} max|dw|="
        f"{np.abs(w.cpu().numpy() - w_ref).max():.2e}")


# ---------------------------------------------------------------- router
# Router scores fused with the route step (MACS §3.1; reading R17).  Shapes:
# the multimodal prefill batch (no H split), the decode batch (8-way split),
# single and ragged token tiles, expert counts that pad to every column width
# (8 -> 32, 60 -> 64, 128, 200 -> 256) and the Mixtral width H = 4096.
ROUTER_CASES = [
    ("prefill_t8192", 8192, 2048, 128, 8, 8, "bf16", 0),
    ("decode_t128", 128, 2048, 128, 8, 8, "bf16", 1),
    ("t1", 1, 2048, 128, 8, 8, "bf16", 2),
    ("t33_ragged", 33, 2048, 128, 8, 8, "bf16", 3),
    ("t2000_split4", 2000, 1024, 128, 8, 8, "bf16", 4),
    ("mixtral_t4096_n8", 4096, 4096, 8, 2, 2, "bf16", 5),
    ("mixtral_t64_n8_r0", 64, 4096, 8, 2, 0, "bf16", 6),
    ("n60_h192", 300, 192, 60, 4, 4, "bf16", 7),
    ("n200", 500, 512, 200, 8, 8, "bf16", 8),
    ("n256_t96", 96, 2048, 256, 8, 8, "bf16", 9),
    ("f32_tiny", 256, 128, 8, 2, 2, "f32", 10),
    ("f32_n128", 77, 256, 128, 8, 8, "f32", 11),
]


@pytest.mark.parametrize("name,T,H,N,k,R,dtype,seed", ROUTER_CASES,
                         ids=[c[0] for c in ROUTER_CASES])
def test_router_topk_parity(name, T, H, N, k, R, dtype, seed):
    """Scores within the summation bound of the fp64 oracle: fp32
    accumulation of H exact bf16 products (or H fused multiply-adds in fp32)
    errs by at most about H * 2^-24 * sum_h |x_h w_h|; twice that is
    allowed.  The ranking is a decision taken on the kernel's own fp32
    scores: the oracle's route over those scores must give the same ids and
    fallbacks bit for bit, and gates within the gate tolerance; moe_route
    over the same scores must give every output bit for bit."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import elem_tensor
    say(f"router top-k {name}: T={T} H={H} N={N} k={k} R={R} {dtype}")
    wl = configs.MM_PREFILL.with_(T=T, H=H, N=N, dtype=dtype)
    x = synth.activations(wl, seed)
    w = synth.router_weights(wl, seed)
    xd, wd = elem_tensor(x, dtype, "cuda"), elem_tensor(w, dtype, "cuda")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ws = B.new_workspace(B.moe_router_workspace_size(T, N, H, tdt), "cuda")
    outs = []
    for rep in range(2):  # the tickets must be back at zero for the second call
        outs.append([None if t is None else t.clone() for t in
                     B.moe_router_topk(xd, wd, k, R, ws)])
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    logits, ids, gates, fb = outs[0]
    z = logits.cpu().numpy()
    ref = O.router_logits(x, w, dtype)
    bound = 2.0 * H * 2.0 ** -24 * (np.abs(O.decode(x, dtype)) @ np.abs(O.decode(w, dtype)).T)
    err = np.abs(z.astype(np.float64) - ref)
    assert (err <= bound + 1e-30).all(), f"max err/bound {np.max(err / (bound + 1e-30)):.3f}"
    r_ids, r_g, r_fb = O.route(z, k, R)
    np.testing.assert_array_equal(ids.cpu().numpy(), r_ids)
    if R:
        np.testing.assert_array_equal(fb.cpu().numpy(), r_fb)
    g = gates.cpu().numpy().astype(np.float64)
    assert (np.abs(g - r_g) <= 1e-7 + 1e-5 * np.abs(r_g)).all()
    s_ids, s_g, s_fb = B.moe_route(logits, k, R)
    assert torch.equal(s_ids, ids) and torch.equal(s_g, gates)
    if R:
        assert torch.equal(s_fb, fb)
    # without the scores output: the same ranking and gates
    _, ids2, g2, fb2 = B.moe_router_topk(xd, wd, k, R, ws, want_logits=False)
    assert torch.equal(ids2, ids) and torch.equal(g2, gates)
    if R:
        assert torch.equal(fb2, fb)
    say(f"max score err / bound {np.max(err / (bound + 1e-30)):.2e}")


# ---------------------------------------------------------------- similarity
# SERE §4.2 calibration (reading R18).  Kernel parity on given matrices:
# the Gram entries are fp32 sums of at most 4096 exact bf16 products, then
# fp64 sums, so |dG_ij| <= 4098 * 2^-24 * sum_k |a_ik a_jk| (fp32 partials
# included); S = G_ij / sqrt(G_ii G_jj) inherits that relative error from
# each factor, plus the final fp32 rounding.  Twice the bound is allowed.
def _sim_bound(v):
    a = np.abs(v)
    e = 4098 * 2.0 ** -24 * (a @ a.T)
    g = v @ v.T
    d = np.sqrt(np.diag(g))
    dn = np.outer(d, d)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = e / np.where(dn > 0, dn, 1.0)
        ed = np.diag(e) / np.where(np.diag(g) > 0, np.diag(g), 1.0)
    return 2.0 * (rel + np.abs(g / np.where(dn > 0, dn, 1.0)) * 0.5 *
                  (ed[:, None] + ed[None, :])) + 2.0 ** -23


SIM_CASES = [
    ("n128_qwen_cal", 128, 256 * 2048, "bf16", 0),
    ("n8_mixtral", 8, 64 * 4096, "bf16", 1),
    ("n60_ragged", 60, 64 * 999, "bf16", 2),
    ("n100_long", 100, 64 * 9001, "bf16", 3),
    ("n33_short", 33, 64 * 3, "bf16", 4),
    ("f32_n8", 8, 300, "f32", 5),
    ("f32_n128", 128, 1000, "f32", 6),
]


@pytest.mark.parametrize("name,N,D,dtype,seed", SIM_CASES, ids=[c[0] for c in SIM_CASES])
def test_expert_similarity_parity(name, N, D, dtype, seed):
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import elem_tensor
    say(f"expert similarity {name}: N={N} D={D} {dtype}")
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((N, D)).astype(np.float32)
    # special rows: a scaled copy, a negated copy, a zero row, and a row
    # correlated with row 0
    v[1] = 0.5 * v[0]
    v[2] = -v[0]
    v[3] = 0.0
    if N > 5:
        v[5] = 0.6 * v[0] + 0.8 * v[4]
    stored = synth.f32_to_bf16_bits(v) if dtype == "bf16" else v
    ref = O.frobenius_similarity(stored, dtype)
    vd = elem_tensor(stored, dtype, "cuda")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ws = B.new_workspace(B.moe_similarity_workspace_size(N, D, tdt), "cuda")
    s1 = B.moe_expert_similarity(vd, ws).cpu().numpy().astype(np.float64)
    s2 = B.moe_expert_similarity(vd, ws).cpu().numpy().astype(np.float64)
    assert (s1 == s2).all()                       # deterministic
    bound = _sim_bound(O.decode(stored, dtype))
    err = np.abs(s1 - ref)
    assert (err <= bound).all(), f"max err/bound {np.max(err / bound):.3f}"
    assert (np.diag(s1) == 1.0).all()
    assert (s1[3, np.arange(N) != 3] == 0.0).all()   # the zero matrix
    say(f"max |dS| {err.max():.2e}")


def test_calibration_pipeline_end_to_end():
    """Calibration activations from the GPU's own FFN (every token through
    every expert: k = N) fed to the similarity kernel, against the oracle's
    fp64 activations.  The GPU rounds h and each output row to bf16
    (relative 2^-9 per element), so the similarities agree to about 1e-3;
    5e-3 absolute is allowed."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd.staging import elem_tensor
    wl = configs.MM_PREFILL.with_(T=64, H=256, N=16, k=4, I=128)
    T, H, N, I = wl.T, wl.H, wl.N, wl.I
    say(f"calibration pipeline T={T} H={H} N={N} I={I}")
    x = synth.activations(wl, 7)
    w13, w2 = synth.expert_weights(wl, 7)
    w13[3], w2[3] = w13[1], w2[1]                 # two identical experts
    ref = O.frobenius_similarity(O.calibration_activations(x, w13, w2, "bf16"), "f64")
    xd, w13d, w2d = (elem_tensor(a, "bf16", "cuda") for a in (x, w13, w2))
    offsets = torch.arange(0, (N + 1) * T, T, dtype=torch.int32, device="cuda")
    row_token = torch.arange(T, dtype=torch.int32, device="cuda").repeat(N)
    h = torch.empty((T * N, I), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T * N, H), dtype=torch.bfloat16, device="cuda")
    B.moe_ffn_gate_up(xd, row_token, offsets, w13d, N, h)
    B.moe_ffn_down(h, offsets, w2d, T, N, out)
    ws = B.new_workspace(B.moe_similarity_workspace_size(N, T * H, torch.bfloat16), "cuda")
    s = B.moe_expert_similarity(out.view(N, T * H), ws).cpu().numpy().astype(np.float64)
    assert np.abs(s - ref).max() <= 5e-3, np.abs(s - ref).max()
    assert s[1, 3] == 1.0 or abs(s[1, 3] - 1.0) < 1e-6   # identical experts
    say(f"max |dS| {np.abs(s - ref).max():.2e}")
