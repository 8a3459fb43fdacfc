"""Benchmark one MoE-layer forward (route -> SERE -> capacity -> dispatch ->
expert FFN -> combine) through the C ABI on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the Qwen3-30B-A3B-shaped decode step at batch 128 with
SERE K'=2, rho=0.5 (T=128, H=2048, N=128, top-8, I=768, bf16).  A step is one
pass of the whole path over one batch; inputs are resident in HBM before the
timed region.  Two copies of the expert weights alternate between steps so
the weight stream is not served from the 256 MB Infinity Cache.

Prints one JSON line: whole-layer tokens/s (value) and µs per decode step,
the roofline of the dominant kernel (the HBM-bound gate-up GEMM), the
whole step's HBM fraction from the per-token byte model, per-kernel
fractions, p10/p50/p90 of the graph-replayed step, the largest
entropy-weighted expert load (the straggler that sets an expert-parallel
layer's latency), and the CPU oracle timed on a bounded sample of the same
workload.  The same line carries the prefill half of the metric
("prefill": the 8192-token multimodal prefill with MACS, tokens/s and the
MFMA fractions of both expert GEMMs), the tiny fp32 layer and the
Mixtral-shaped decode and prefill layers (also with re-routing off, R = 0:
capacity plus drop only), each timed in its own regions.  --only times the
named workload alone.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 157.3
METRIC = ("MoE-layer tokens/s (prefill) + decode-step µs at B=128; "
          "% of HBM/MFMA peak")

# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc runs
# of this script on one MI355X (FETCH_SIZE, then WRITE_SIZE: KiB per
# dispatch, mean over the dispatches of the run), each scaled by what the
# same counter reads for a plain 256 MiB device-to-device copy
# (`--copy-probe-mib 256`: FETCH_SIZE reads 128 MiB -> x2.0, WRITE_SIZE
# reads 256 MiB -> x1.0).  A reading holds only for the kernel sources it was
# taken on (sha256 over GEMM_SOURCES); otherwise traffic is reported as null.
GEMM_SOURCES = ("mixture_experts_layer_macs_amd/csrc/ffn.hip",
                "mixture_experts_layer_macs_amd/csrc/common.h",
                "mixture_experts_layer_macs_amd/csrc/dma.h")
DIFF_REPS = 5  # timed-region pairs per in-step kernel duration

HBM_COUNTERS = {
    "qwen3_decode_b128": dict(
        kernel="gate_up_swiglu", fetch_kib=130582.0, write_kib=1536.8,
        fetch_scale=2.0, write_scale=1.0,
        sources_sha256="8e2ed701da26d2d73f0aec77c63fc73244d0d78776e312c687ff4042c12f5457"),
}


def counted_traffic(workload):
    """Scaled HBM bytes per launch of the dominant kernel, or None when no
    reading exists for this workload or the kernel has changed since."""
    import hashlib
    rec = HBM_COUNTERS.get(workload)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(rec["fetch_kib"] * 1024 * rec["fetch_scale"] +
               rec["write_kib"] * 1024 * rec["write_scale"])


def hold_gpu(seconds):
    """Occupy the current stream for about `seconds` (a spin kernel), so the
    host can queue work behind it."""
    import torch
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(seconds * 2.5e9))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="qwen3_decode_b128")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--copies", type=int, default=2,
                   help="weight copies rotated between steps")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the HIP-graph timed region")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only copy a buffer of this many MiB device to device "
                        "three times and exit (calibrates HBM byte counters)")
    p.add_argument("--sweep", action="store_true",
                   help="the 48-layer decode sweep: batch x visual fraction x "
                        "SERE setting, one JSON line with the whole table")
    p.add_argument("--layers", type=int, default=48)
    p.add_argument("--batches", default="1,8,32,64,128,256",
                   help="sweep: batch sizes (comma-separated)")
    p.add_argument("--fracs", default="0.1,0.5,0.9",
                   help="sweep: visual fractions (comma-separated)")
    p.add_argument("--kprimes", default="0,1,2",
                   help="sweep: SERE settings K' (0 = off; comma-separated)")
    p.add_argument("--entropy", action="store_true",
                   help="time the entropy-weight producer on the multimodal "
                        "prefill batch (T=8192, H=2048, bf16) and exit")
    p.add_argument("--router", action="store_true",
                   help="time the router scores fused with top-k on the "
                        "prefill (T=8192) and decode (T=128) batches and exit")
    p.add_argument("--similarity", action="store_true",
                   help="time the SERE similarity calibration of one layer "
                        "(256 calibration tokens through all 128 experts, then "
                        "the Frobenius similarity) and exit")
    p.add_argument("--only", action="store_true",
                   help="time the named workload alone (by default the "
                        "decode headline also times the 8192-token multimodal "
                        "prefill, the tiny fp32 layer and the Mixtral-shaped "
                        "layers)")
    p.add_argument("--weights", choices=("panels", "rows"), default="panels",
                   help="bf16 expert weights in the panel layout written once "
                        "by moe_pack_weights (default), or in the row layout")
    p.add_argument("--separate-routing", action="store_true",
                   help="route with the four separate calls instead of the "
                        "single fused launch")
    return p.parse_args()


def cpu_baseline(inp, budget_s):
    """The oracle, untuned, over whole steps of the same workload until the
    time budget is used (at least one step)."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = os.cpu_count() or 1
    t0 = time.perf_counter()
    n = 0
    t_route = t_ffn = 0.0
    while True:
        a = time.perf_counter()
        rt = O.layer_routing(inp)
        b = time.perf_counter()
        O.layer_outputs(inp, rt)
        c = time.perf_counter()
        t_route += b - a
        t_ffn += c - b
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return dict(value=round(n * inp["T"] / el, 3), unit="tokens/s",
                cores=int(blas), kind="oracle",
                cores_detail=dict(routing_threads=1, ffn_blas_threads=int(blas),
                                  os_cpu_count=os.cpu_count(),
                                  affinity=int(affinity)),
                routing_s_per_step=round(t_route / n, 4),
                ffn_s_per_step=round(t_ffn / n, 4),
                sample=(f"{n} full layer step(s) of the same workload "
                        f"(T={inp['T']}): routing {t_route / n:.3f} s/step "
                        f"single-threaded Python, FFN+combine "
                        f"{t_ffn / n:.3f} s/step fp64 numpy on "
                        f"{int(blas)} BLAS threads"))



def run_sweep(args):
    """48 MoE layers of the Qwen3-30B-A3B shape (T <= 256, H 2048, N 128,
    top-8, I 768, bf16), each with its own seeded router logits (Zipf
    popularity permutation), similarity and protection matrices (16
    protected experts) and random-init expert weights; MACS gamma 1.25,
    lam 1, R 8.  For every point of batch x visual fraction x SERE setting
    the whole 48-layer step is captured in one HIP graph and replayed."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd import configs, synth
    from mixture_experts_layer_macs_amd.staging import elem_tensor, to_device
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = configs.SWEEP_LAYER
    H, N, k, I, R = base.H, base.N, base.k, base.I, base.R
    L = args.layers
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    print(f"[sweep] random-init weights for {L} layers on the GPU", file=sys.stderr,
          flush=True)
    w13 = [torch.empty((N, 2 * I, H), dtype=torch.bfloat16, device=dev).normal_(
        0.0, 0.02, generator=gen) for _ in range(L)]
    w2 = [torch.empty((N, H, I), dtype=torch.bfloat16, device=dev).normal_(
        0.0, 0.02, generator=gen) for _ in range(L)]
    panels = args.weights == "panels"
    if panels:  # packed once per layer, as at model load
        for l in range(L):
            w13[l], w2[l] = B.moe_pack_weights(w13[l], w2[l])
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    rows = []
    for T in [int(v) for v in args.batches.split(",")]:
        x = elem_tensor(synth.activations(base.with_(T=T), args.seed), "bf16", dev)
        lay = B.Layer(T, H, N, k, I, R, torch.bfloat16, dev)
        ws = B.new_workspace(B.moe_ffn_combine_workspace_size(T, N, k, H, I, torch.bfloat16),
                             dev)
        for frac in [float(v) for v in args.fracs.split(",")]:
            for kp in [int(v) for v in args.kprimes.split(",")]:
                wl = base.with_(T=T, visual=f"frac:{frac}", kprime=kp)
                inps = [to_device(synth.make_inputs(wl, args.seed, layer=l,
                                                    weights=False), dev, weights=False)
                        for l in range(L)]

                def layer(l):
                    d = inps[l]
                    lay.routing(d["logits"], d["is_visual"], d["entropy_w"],
                                d["modality"], d["sim"], d["prot"], kp, wl.rho,
                                wl.gamma, wl.lam, wl.group)
                    B.moe_expert_ffn_combine(x, lay.disp["row_token"],
                                             lay.disp["expert_offsets"], w13[l], w2[l],
                                             lay.disp["slot_row"], lay.topk_gates, k, ws,
                                             lay.out_rows, lay.y, panels=panels)

                # union sizes and weight bytes, layer by layer (untimed)
                ub = us = uf = 0
                for l in range(L):
                    layer(l)
                    torch.cuda.synchronize()
                    ub += int(torch.unique(lay.topk_ids).numel())
                    us += int(torch.unique(lay.slot_sere if kp else lay.topk_ids).numel())
                    uf += int((torch.diff(lay.disp["expert_offsets"]) > 0).sum().item())
                g = torch.cuda.CUDAGraph()
                cs = torch.cuda.Stream()
                with torch.cuda.graph(g, stream=cs):
                    for l in range(L):
                        layer(l)
                for _ in range(2):
                    g.replay()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                reps = max(3, args.steps // 10)
                e0.record()
                for _ in range(reps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                wbytes = uf * 3 * H * I * 2
                rows.append(dict(batch=T, visual_frac=frac,
                                 sere="off" if kp == 0 else f"K'={kp}",
                                 union_baseline=round(ub / L, 2),
                                 union_sere=round(us / L, 2),
                                 union_final=round(uf / L, 2),
                                 weight_GB_per_step=round(wbytes / 1e9, 3),
                                 us_per_step=round(ms * 1e3, 1),
                                 weight_GBps=round(wbytes / (ms * 1e-3) / 1e9, 1)))
                print(f"[sweep] {rows[-1]}", file=sys.stderr, flush=True)
                del g, inps
    print(json.dumps({"metric": "48-layer decode sweep: union size, weight bytes "
                                "moved and us per 48-layer step",
                      "unit": "us", "higher_is_better": False, "n_gpus": 1,
                      "layers": L, "dtype": "bf16",
                      "weights": "panels" if panels else "rows",
                      "data": "synthetic (seeded; random-init weights)",
                      "config": {"workload": "sweep_layer x 48", "H": H, "N": N,
                                 "k": k, "I": I, "gamma": base.gamma,
                                 "lam": base.lam, "R": R, "rho": base.rho},
                      "sweep": rows}), flush=True)


def run_entropy(args):
    """Entropy-weight producer (MACS §3.2 Eq. 4-5) on the 8192-token
    multimodal prefill batch: one read of every token row, HBM-bound."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd import configs, synth
    from mixture_experts_layer_macs_amd.staging import elem_tensor
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = configs.MM_PREFILL
    T, H = wl.T, wl.H
    xs = [elem_tensor(synth.visual_features(T, H, "bf16", args.seed + c), "bf16", dev)
          for c in range(2)]
    vis = torch.from_numpy(synth.visual_mask(wl, args.seed)).to(dev)
    ws = B.new_workspace(B.moe_entropy_workspace_size(T), dev)
    w = torch.empty(T, dtype=torch.float32, device=dev)
    for i in range(args.warmup):
        B.moe_entropy_weights(xs[i % 2], vis, 1.0, 1e-6, ws, w)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        B.moe_entropy_weights(xs[i % 2], vis, 1.0, 1e-6, ws, w)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = T * H * 2 + T * (1 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "entropy-weight producer throughput",
                      "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
                      "us_per_call": round(ms * 1e3, 2), "n_gpus": 1,
                      "dtype": "bf16", "data": "synthetic (seeded)",
                      "config": {"workload": "entropy_t8192_h2048", "T": T, "H": H},
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "bytes_per_launch": nbytes}}), flush=True)

def run_router(args):
    """Router scores fused with the route step (MACS §3.1): the multimodal
    prefill batch (T=8192) and the decode batch (T=128), H=2048, N=128,
    top-8 with R=8 fallbacks, bf16, scores not written out.  Eight copies
    of x and W_g rotate between calls so that the stream is not served from
    the 256 MB Infinity Cache.  HBM-bound: one read of x and W_g plus the
    routing outputs."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd import configs, synth
    from mixture_experts_layer_macs_amd.staging import elem_tensor
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    res = {}
    for name, T in (("prefill_t8192", 8192), ("decode_t128", 128)):
        wl = configs.MM_PREFILL.with_(T=T)
        H, N, k, R = wl.H, wl.N, wl.k, wl.R
        xs = [elem_tensor(synth.activations(wl, args.seed + c), "bf16", dev) for c in range(8)]
        wsg = [elem_tensor(synth.router_weights(wl, args.seed + c), "bf16", dev) for c in range(8)]
        ws = B.new_workspace(B.moe_router_workspace_size(T, N, H, torch.bfloat16), dev)
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        g = torch.empty((T, k), dtype=torch.float32, device=dev)
        fb = torch.empty((T, R), dtype=torch.int32, device=dev)

        def call(i):
            B.moe_router_topk(xs[i % 8], wsg[i % 8], k, R, ws, topk_ids=ids,
                              topk_gates=g, fallback_ids=fb, want_logits=False)
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        hold_gpu(0.02)
        e0.record()
        for i in range(args.steps):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        nbytes = T * H * 2 + N * H * 2 + T * k * 8 + T * R * 4
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = dict(T=T, us_per_call=round(us, 2),
                         tokens_per_s=round(T / (us * 1e-6), 1),
                         bytes_per_call=nbytes, GBps=round(gbs, 1),
                         hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        print(f"[router] {name}: {res[name]}", file=sys.stderr, flush=True)
    p = res["prefill_t8192"]
    print(json.dumps({"metric": "router scores + top-k throughput",
                      "value": p["tokens_per_s"], "unit": "tokens/s",
                      "us_per_call": p["us_per_call"], "n_gpus": 1,
                      "dtype": "bf16", "data": "synthetic (seeded)",
                      "config": {"workload": "router_t8192_h2048_n128", "T": 8192,
                                 "H": 2048, "N": 128, "k": 8, "R": 8},
                      "roofline": {"bound": "hbm", "achieved": p["GBps"],
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": p["hbm_frac"],
                                   "bytes_per_launch": p["bytes_per_call"]},
                      "decode_t128": res["decode_t128"]}), flush=True)


def run_similarity(args):
    """SERE similarity calibration (SERE §4.2) for one layer of the qwen3
    shape (N=128, H=2048, I=768, bf16): a calibration batch of 256
    synthetic tokens goes through every expert (the grouped FFN with k = N,
    32768 rows), then the Frobenius similarity of the 128 activation
    matrices [256 x 2048] is formed.  Three copies of the activations
    rotate between similarity calls so the 128 MB are not served from the
    Infinity Cache; the similarity step is HBM-bound."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd import configs, synth
    from mixture_experts_layer_macs_amd.staging import elem_tensor
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = configs.QWEN3_DECODE.with_(T=256)
    T, H, N, I = wl.T, wl.H, wl.N, wl.I
    x = elem_tensor(synth.activations(wl, args.seed), "bf16", dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    w13 = torch.empty((N, 2 * I, H), dtype=torch.bfloat16, device=dev).normal_(0.0, 0.02, generator=gen)
    w2 = torch.empty((N, H, I), dtype=torch.bfloat16, device=dev).normal_(0.0, 0.02, generator=gen)
    offsets = torch.arange(0, (N + 1) * T, T, dtype=torch.int32, device=dev)
    row_token = torch.arange(T, dtype=torch.int32, device=dev).repeat(N)
    h = torch.empty((T * N, I), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty((T * N, H), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    D = T * H
    ws = B.new_workspace(B.moe_similarity_workspace_size(N, D, torch.bfloat16), dev)
    sim = torch.empty((N, N), dtype=torch.float32, device=dev)

    def ffn(i):
        B.moe_ffn_gate_up(x, row_token, offsets, w13, N, h)
        B.moe_ffn_down(h, offsets, w2, T, N, outs[i % 3])

    def simc(i):
        B.moe_expert_similarity(outs[i % 3].view(N, D), ws, sim)
    for i in range(3):
        ffn(i)
    torch.cuda.synchronize()

    def timed(fn, n):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        hold_gpu(0.02)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3
    us_sim = timed(simc, args.steps)
    us_ffn = timed(ffn, max(5, args.steps // 5))
    nbytes = N * D * 2 + N * N * 4
    gbs = nbytes / (us_sim * 1e-6) / 1e9
    print(json.dumps({"metric": "SERE similarity calibration: Frobenius similarity of the experts' calibration activations",
                      "value": round(us_sim, 2), "unit": "us per layer (similarity step)",
                      "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
                      "data": "synthetic (seeded calibration tokens, random-init experts)",
                      "config": {"workload": "similarity_n128_t256_h2048", "N": N, "T_cal": T,
                                 "H": H, "I": I},
                      "ffn_all_experts_us": round(us_ffn, 1),
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "bytes_per_launch": nbytes}}), flush=True)


def _q(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def measure(wl, args, with_cpu=False):
    """Time one workload: a step is one pass of route -> SERE -> capacity ->
    dispatch -> gate-up -> down -> combine over one batch, inputs resident
    in HBM.  Returns a dict of step times, in-step kernel times, routing
    statistics and roofline figures."""
    import torch
    from mixture_experts_layer_macs_amd import binding as B
    from mixture_experts_layer_macs_amd import synth
    from mixture_experts_layer_macs_amd.staging import to_device, torch_elem_dtype

    dev = torch.device("cuda:0")
    print(f"[bench] {wl.name}: generating inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl, args.seed)
    d = to_device(inp, dev)
    w13s = [d["w13"]] + [d["w13"].clone() for _ in range(args.copies - 1)]
    w2s = [d["w2"]] + [d["w2"].clone() for _ in range(args.copies - 1)]
    # weights packed once, as at model load; the step reads only the packs
    panels = wl.dtype == "bf16" and args.weights == "panels"
    if panels:
        packed = [B.moe_pack_weights(a, b) for a, b in zip(w13s, w2s)]
        w13s, w2s = [p[0] for p in packed], [p[1] for p in packed]
        del packed
        d["w13"] = d["w2"] = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    T, H, N, k, I, R = wl.T, wl.H, wl.N, wl.k, wl.I, wl.R
    lay = B.Layer(T, H, N, k, I, R, torch_elem_dtype(wl.dtype), dev)
    h = torch.empty((T * k, I), dtype=torch_elem_dtype(wl.dtype), device=dev)
    decode = wl.kprime > 0 or T * k <= 32 * N
    fused = lay.can_fuse and not args.separate_routing
    steps = args.steps if decode else max(5, args.steps // 2)

    def gate_up(i):
        B.moe_ffn_gate_up(d["x"], lay.disp["row_token"],
                          lay.disp["expert_offsets"], w13s[i % len(w13s)], k, h,
                          panels=panels)

    # decode batches of at most 16 dispatch rows on packed weights whose down
    # half runs as a GEMV (I / 256 in 1, 2, 3, 4, 8): the combine is folded
    # into it (moe_ffn_down_combine), so "down" below times both
    fold = (panels and decode and T * k <= 16 and I % 256 == 0
            and I // 256 in (1, 2, 3, 4, 8))
    ws_comb = (B.new_workspace(B.moe_ffn_combine_workspace_size(
        T, N, k, H, I, torch_elem_dtype(wl.dtype)), dev) if fold else None)

    def down(i):
        if fold:
            B.moe_ffn_down_combine(h, lay.disp["row_token"], lay.disp["expert_offsets"],
                                   w2s[i % len(w2s)], lay.disp["slot_row"],
                                   lay.topk_gates, T, k, ws_comb, lay.out_rows, lay.y,
                                   panels=panels)
        else:
            B.moe_ffn_down(h, lay.disp["expert_offsets"], w2s[i % len(w2s)], T, k,
                           lay.out_rows, panels=panels)

    def step(i, skip=()):
        lay.routing(d["logits"], d["is_visual"], d["entropy_w"], d["modality"],
                    d["sim"], d["prot"], wl.kprime, wl.rho, wl.gamma, wl.lam,
                    wl.group, fused=fused)
        if "gate_up" not in skip:
            gate_up(i)
        if "down" not in skip:
            down(i)
        if not fold:
            B.moe_combine(lay.out_rows, lay.disp["slot_row"], lay.topk_gates, lay.y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph_cache = {}

    def graphs_for(skip):
        if skip not in graph_cache:
            gs = []
            cap_stream = torch.cuda.Stream()
            for c in range(len(w13s)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap_stream):
                    step(c, skip)
                gs.append(g)
            graph_cache[skip] = gs
        return graph_cache[skip]

    def timed(skip=(), graph=False, per_step=False):
        """Mean ms per step over `steps` steps with HIP events at the two ends
        of the region (and, with per_step, one event between replays).
        Eager: a spin kernel holds the stream while the host queues the
        steps, so they then run back to back.  Graph: the step is captured
        once per weight copy and replayed."""
        ev = [torch.cuda.Event(enable_timing=True)
              for _ in range(steps + 1 if per_step else 2)]
        if graph:
            gs = graphs_for(skip)
            for i in range(args.warmup):
                gs[i % len(gs)].replay()
            torch.cuda.synchronize()
            ev[0].record()
            for i in range(steps):
                gs[i % len(gs)].replay()
                if per_step:
                    ev[i + 1].record()
            ev[-1].record()
        else:
            torch.cuda.synchronize()
            hold_gpu(steps * 1e-4 + 2e-3)
            ev[0].record()
            for i in range(steps):
                step(i, skip)
            ev[-1].record()
        torch.cuda.synchronize()
        if per_step:
            return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return ev[0].elapsed_time(ev[-1]) / steps

    print(f"[bench] {wl.name}: timed steps", file=sys.stderr, flush=True)
    t_wall = time.perf_counter()
    eager_ms = timed()
    t_wall = time.perf_counter() - t_wall
    per_step = None if args.no_graph else timed(graph=True, per_step=True)
    graph_ms = None if per_step is None else float(np.mean(per_step))
    use_graph = not args.no_graph

    # In-step duration of each expert GEMM: the step time minus the time of
    # the same step with that kernel left out (same timing mode), the median
    # over DIFF_REPS alternating pairs of timed regions.  An event pair around
    # one launch would add the dispatch gap after the first event.
    def in_step_ms(name):
        return float(np.median([timed((), use_graph) - timed((name,), use_graph)
                                for _ in range(DIFF_REPS)]))
    gu_ms = in_step_ms("gate_up")
    dn_ms = in_step_ms("down")

    off = lay.disp["expert_offsets"].cpu().numpy()
    counts = np.diff(off)
    M = int(off[-1])
    U = int((counts > 0).sum())
    el = 2 if wl.dtype == "bf16" else 4
    stats = lay.cap["stats"].cpu().numpy()
    load_q = lay.cap["load_q"].cpu().numpy().astype(np.float64) / 65536.0
    topk = lay.topk_ids.cpu().numpy()
    slot_sere = (lay.slot_sere if wl.kprime else lay.topk_ids).cpu().numpy()
    best_ms = eager_ms if graph_ms is None else min(eager_ms, graph_ms)
    out = dict(
        workload=wl.name, T=T, H=H, N=N, k=k, I=I, dtype=wl.dtype,
        step_us=round(best_ms * 1e3, 2),
        tokens_per_s=round(T / (best_ms * 1e-3), 1),
        eager_us=round(eager_ms * 1e3, 2),
        graph_us=None if graph_ms is None else round(graph_ms * 1e3, 2),
        mode="eager" if graph_ms is None or eager_ms <= graph_ms else "hip-graph",
        steps=steps,
        routing="fused" if fused else "separate",
        combine="folded into down" if fold else "separate",
        weights="panels" if panels else "rows",
        union_baseline=int(len(np.unique(topk))),
        union_sere=int(len(np.unique(slot_sere))),
        union_final=U, kept_rows=M,
        dropped=int(stats[2]), macs_rerouted=int(stats[3]),
        # Eq. 2 straggler proxy: the largest entropy-weighted expert load
        max_load_tokens=round(float(load_q.max()), 4),
        mean_active_load_tokens=round(float(load_q[load_q > 0].mean()), 4)
        if (load_q > 0).any() else 0.0,
        kernels_us={"gate_up_swiglu": round(gu_ms * 1e3, 2),
                    "down": round(dn_ms * 1e3, 2),
                    "routing_combine_and_gaps": round((best_ms - gu_ms - dn_ms) * 1e3, 2)},
        wall_s=round(t_wall, 3),
    )
    if per_step is not None:
        out["graph_step_us_p10_p50_p90"] = [round(_q(per_step, q) * 1e3, 2)
                                           for q in (10, 50, 90)]
    if decode:
        # algorithmic bytes: every active expert's weights once, x once per
        # token, h written by gate-up and read by down, out rows
        gu_bytes = U * 2 * I * H * el + T * H * el + M * I * el
        dn_bytes = U * H * I * el + M * I * el + M * H * el
        step_bytes = (U * 3 * H * I * el + 2 * T * H * el + T * N * 4
                      + (N * N * 5 if wl.kprime else 0))
        gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
        out["roofline"] = dict(
            bound="hbm", achieved=round(gbs(gu_bytes, gu_ms), 1),
            peak=HBM_PEAK_GBS, unit="GB/s",
            frac=round(gbs(gu_bytes, gu_ms) / HBM_PEAK_GBS, 4),
            traffic=counted_traffic(wl.name), kernel="gate_up_swiglu",
            kernel_us=round(gu_ms * 1e3, 2), bytes_per_launch=int(gu_bytes))
        out["kernels_roofline"] = {
            "gate_up_swiglu": dict(GBps=round(gbs(gu_bytes, gu_ms), 1),
                                   frac=round(gbs(gu_bytes, gu_ms) / HBM_PEAK_GBS, 4),
                                   bytes=int(gu_bytes)),
            "down": dict(GBps=round(gbs(dn_bytes, dn_ms), 1),
                         frac=round(gbs(dn_bytes, dn_ms) / HBM_PEAK_GBS, 4),
                         bytes=int(dn_bytes))}
        out["step_roofline"] = dict(
            bound="hbm", bytes_per_step=int(step_bytes),
            achieved=round(gbs(step_bytes, best_ms), 1), peak=HBM_PEAK_GBS,
            unit="GB/s", frac=round(gbs(step_bytes, best_ms) / HBM_PEAK_GBS, 4),
            bytes_model="union_final*3*H*I*el + 2*T*H*el + T*N*4 (+ N*N*5 with SERE)")
    else:
        peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_VALU_PEAK_TFLOPS
        bound = "mfma" if wl.dtype == "bf16" else "alu"
        gu_fl, dn_fl = 4.0 * M * H * I, 2.0 * M * H * I
        tf = lambda f, ms: f / (ms * 1e-3) / 1e12
        out["roofline"] = dict(
            bound=bound, achieved=round(tf(gu_fl, gu_ms), 2), peak=peak,
            unit="TFLOP/s", frac=round(tf(gu_fl, gu_ms) / peak, 4),
            traffic=counted_traffic(wl.name), kernel="gate_up_swiglu",
            kernel_us=round(gu_ms * 1e3, 2), flops_per_launch=gu_fl)
        out["kernels_roofline"] = {
            "gate_up_swiglu": dict(TFLOPs=round(tf(gu_fl, gu_ms), 2),
                                   frac=round(tf(gu_fl, gu_ms) / peak, 4),
                                   flops=gu_fl),
            "down": dict(TFLOPs=round(tf(dn_fl, dn_ms), 2),
                         frac=round(tf(dn_fl, dn_ms) / peak, 4), flops=dn_fl)}
        out["step_roofline"] = dict(
            bound=bound, flops_per_step=gu_fl + dn_fl,
            achieved=round(tf(gu_fl + dn_fl, best_ms), 2), peak=peak,
            unit="TFLOP/s", frac=round(tf(gu_fl + dn_fl, best_ms) / peak, 4))
    if with_cpu and not args.no_cpu_baseline:
        print(f"[bench] {wl.name}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    del graph_cache, w13s, w2s, d, lay, h
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def _brief(m):
    keys = ("step_us", "tokens_per_s", "graph_step_us_p10_p50_p90", "kernels_us",
            "kernels_roofline", "step_roofline", "union_baseline", "union_sere",
            "union_final", "kept_rows", "dropped", "macs_rerouted",
            "max_load_tokens", "mean_active_load_tokens", "mode", "routing", "combine")
    return {"workload": m["workload"], **{k: m[k] for k in keys if k in m}}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.sweep:
        run_sweep(args)
        return
    if args.entropy:
        run_entropy(args)
        return
    if args.router:
        run_router(args)
        return
    if args.similarity:
        run_similarity(args)
        return
    import torch
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return
    from mixture_experts_layer_macs_amd import build as _build
    if not os.path.exists(_build.LIB):
        _build.build()
    from mixture_experts_layer_macs_amd import configs
    torch.cuda.set_device(0)

    wl = configs.WORKLOADS[args.workload]
    head = measure(wl, args, with_cpu=True)
    res = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(head["step_us"] * 1e-3, 5),
        "step_us": head["step_us"],
        "eager_ms_per_step": round(head["eager_us"] * 1e-3, 5),
        "graph_ms_per_step": (None if head["graph_us"] is None
                              else round(head["graph_us"] * 1e-3, 5)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; random-init weights of the stated shape)",
        "config": {
            "workload": wl.name, "T": wl.T, "H": wl.H, "N": wl.N, "k": wl.k,
            "I": wl.I, "kprime": wl.kprime, "rho": wl.rho,
            "gamma": "inf" if math.isinf(wl.gamma) else wl.gamma, "R": wl.R,
            "union_baseline": head["union_baseline"],
            "union_sere": head["union_sere"], "union_final": head["union_final"],
            "kept_rows": head["kept_rows"], "dropped": head["dropped"],
            "macs_rerouted": head["macs_rerouted"],
            "weight_copies": args.copies, "routing": head["routing"],
            "combine": head["combine"], "mode": head["mode"],
        },
        "roofline": head["roofline"],
        "step_roofline": head["step_roofline"],
        "kernels_roofline": head["kernels_roofline"],
        "kernels_ms": {k: round(v * 1e-3, 4) for k, v in head["kernels_us"].items()},
        "graph_step_us_p10_p50_p90": head.get("graph_step_us_p10_p50_p90"),
        "max_load_tokens": head["max_load_tokens"],
        "mean_active_load_tokens": head["mean_active_load_tokens"],
        "wall_s": head["wall_s"],
        "cpu_baseline": head.get("cpu_baseline"),
    }
    if args.workload == "qwen3_decode_b128" and not args.only:
        # the prefill half of the metric and the other workloads, each its
        # own timed regions after the headline ones
        others = [("prefill", configs.MM_PREFILL),
                  ("tiny_f32", configs.TINY_F32),
                  ("mixtral_decode_t64", configs.MIXTRAL_DECODE),
                  ("mixtral_prefill_t4096", configs.MIXTRAL_PREFILL),
                  ("mixtral_prefill_t4096_drop_only",
                   configs.MIXTRAL_PREFILL.with_(name="mixtral_prefill_t4096_r0",
                                                 R=0))]
        for key, owl in others:
            res[key] = _brief(measure(owl, args))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
